// ensure_experts on the device: the global LRU remap of one layer's routed experts
// onto the slot pool, done by a single 1024-thread workgroup out of LDS.
//
// FreeToken MoE benchmark guide §4.1 and §4.3, FreeToken architecture walk-through
// §5: experts are named by the flat id layer * E + expert; one slot pool serves
// every layer; a step remaps its routed experts with a global LRU policy and the
// missing ones are then copied in.
//
// Batch rules (the pages give the policy, not the batch order):
//   U    = sorted distinct flat ids of the step
//   hits = members of U already owning a slot; misses = the rest, ascending
//   victims: slots not holding a member of U, ordered by the key
//            (not empty, stamp, owner, slot) - the i-th miss takes the i-th
//   |U| > S fails with OES_ERR_CAPACITY and writes nothing to the table
//   on success clock += 1 and every slot holding a member of U gets the clock.
// Hybrid steps (FreeToken MoE benchmark guide §5.4, ensure_experts_hybrid): only
//   the first `take` misses (ascending) are installed, take = min(cap, misses,
//   slots not holding a member of U); the others keep no slot, their requests
//   map to -1 (the CPU executor's share) and they are not stamped; no capacity
//   error.  cap = max_fetch if >= 0, else rint(misses x min(1, fraction)) in
//   double (round half to even) if fraction >= 0, else 1.
//
// Layout in LDS (E <= 4096, S <= 4096):
//   req[E]   u8   expert e of this layer requested
//   emap[E]  i32  slot owning expert e of this layer, or -1
//   mrank[E] i32  rank of expert e among the misses (exclusive scan)
//   khi/klo[Spad] u64  victim keys, bitonic-sorted ascending (keys live in
//                      registers during the sort; LDS is the exchange buffer for
//                      partners 64..kThreads-1 apart); members of U and padding
//                      get the all-ones key and sort last.  For up to 256
//                      candidates (16 * registers per thread * misses) the
//                      first `take` keys come from ranks instead (rank_victims),
//                      with the keys as (hi, lo) pairs over the same bytes.
// Key encoding: khi = (owner != -1) << 63 | stamp  (stamps < 2^62),
//               klo = (owner + 1) << 12 | slot     (owner < 2^50, slot < 4096).

#include <math.h>

#include "oes_internal.h"

namespace oes {

namespace {

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = OES_MAX_EXPERTS / kThreads;  // 4 experts per thread in the scan
constexpr uint64_t kMax = ~0ull;

// Block-wide exclusive scan of one int per thread; returns the exclusive prefix, *total the sum.
__device__ int block_exclusive_scan(int v, int *wave_tot, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      int t = wave_tot[w];
      wave_tot[w] = run;
      run += t;
    }
    wave_tot[kWaves] = run;
  }
  __syncthreads();
  int excl = wave_tot[wave] + inc - v;
  *total = wave_tot[kWaves];
  __syncthreads();
  return excl;
}

__device__ inline bool key_less(uint64_t ah, uint64_t al, uint64_t bh, uint64_t bl) {
  return ah < bh || (ah == bh && al < bl);
}

__device__ inline uint64_t shfl_xor_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Compare-exchange of element i (key a) against its partner (key b) in a
// bitonic stage: keep the smaller key if i is the lower element of an
// ascending pair or the upper element of a descending pair, else the larger.
__device__ inline void keep(uint64_t &ah, uint64_t &al, uint64_t bh, uint64_t bl, bool take_min) {
  const bool b_less = key_less(bh, bl, ah, al);
  if (b_less == take_min) {
    ah = bh;
    al = bl;
  }
}

// Bitonic sort (ascending) of Spad keys held R per thread: element i lives in
// thread i % kThreads, register i / kThreads.  Partners closer than 64 are in
// the same wave (cross-lane shuffle, no barrier); partners kThreads or more
// apart are in the same thread; the rest go through LDS (xh / xl).
template <int R>
__device__ void bitonic_regs(uint64_t (&hi)[R], uint64_t (&lo)[R], int Spad, uint64_t *xh, uint64_t *xl) {
  const int tid = threadIdx.x;
  for (int kk = 2; kk <= Spad; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j >= kThreads) {
        const int rj = j / kThreads;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int p = r ^ rj;
          if (p > r && p < R) {
            const int i = tid + r * kThreads;
            const bool asc = (i & kk) == 0;
            if (key_less(hi[p], lo[p], hi[r], lo[r]) == asc) {
              const uint64_t th = hi[r], tl = lo[r];
              hi[r] = hi[p]; lo[r] = lo[p];
              hi[p] = th; lo[p] = tl;
            }
          }
        }
      } else if (j >= 64) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          xh[tid + r * kThreads] = hi[r];
          xl[tid + r * kThreads] = lo[r];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = tid + r * kThreads;
          const int p = i ^ j;
          keep(hi[r], lo[r], xh[p], xl[p], ((i & j) == 0) == ((i & kk) == 0));
        }
        __syncthreads();
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = tid + r * kThreads;
          const uint64_t ph = shfl_xor_u64(hi[r], j), pl = shfl_xor_u64(lo[r], j);
          keep(hi[r], lo[r], ph, pl, ((i & j) == 0) == ((i & kk) == 0));
        }
      }
    }
  }
}

// Victim keys of the slots (members of U and padding get the all-ones key),
// sorted ascending into khi / klo.
template <int R>
__device__ void sort_victims(const LruArgs &a, const uint8_t *req, int64_t base, uint64_t *khi, uint64_t *klo) {
  uint64_t hi[R], lo[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int s = threadIdx.x + r * kThreads;
    hi[r] = kMax;
    lo[r] = kMax;
    if (s < a.S) {
      const int64_t o = a.owner[s];
      const bool in_u = o >= base && o < base + a.E && req[(int)(o - base)];
      if (!in_u) {
        hi[r] = ((o != -1) ? (1ull << 63) : 0ull) | a.stamp[s];
        lo[r] = ((uint64_t)(o + 1) << 12) | (uint64_t)s;
      }
    }
  }
  bitonic_regs<R>(hi, lo, a.Spad, khi, klo);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = threadIdx.x + r * kThreads;
    if (i < a.Spad) {
      khi[i] = hi[r];
      klo[i] = lo[r];
    }
  }
  __syncthreads();
}

// The m smallest victim keys, ascending, into khi / klo[0..m), by ranks.  Group g
// is the 64 keys of one wave and register r (slots r*kThreads + 64w + lane);
// (1) each key's rank within its group (64 broadcast LDS reads per key); a key
// among the m smallest of the pool is among the m smallest of its group, so
// the keys of group rank < m (at most m per group) are the candidates;
// (2) each candidate's rank among the candidates, counted by kThreads / C
// threads per candidate; rank r < m goes to position r.  Keys are unique (the
// slot is in the low bits) and padding / members of U never become
// candidates; m <= slots not holding a member of U (the capacity check), so
// positions 0..m-1 are all filled.  Needs 16 * R * m <= kRankCand.
constexpr int kRankCand = 256;

template <int R>
__device__ void rank_victims(const LruArgs &a, const uint8_t *req, int64_t base, int m, uint64_t *khi,
                             uint64_t *klo, u64x2 *kpair, uint64_t *cand_h, uint64_t *cand_l, int *cnt) {
  const int tid = threadIdx.x, wave = tid >> 6;
  uint64_t hi[R], lo[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int s = tid + r * kThreads;
    hi[r] = kMax;
    lo[r] = kMax;
    if (s < a.S) {
      const int64_t o = a.owner[s];
      const bool in_u = o >= base && o < base + a.E && req[(int)(o - base)];
      if (!in_u) {
        hi[r] = ((o != -1) ? (1ull << 63) : 0ull) | a.stamp[s];
        lo[r] = ((uint64_t)(o + 1) << 12) | (uint64_t)s;
      }
    }
    kpair[s] = u64x2{hi[r], lo[r]};
  }
  const int C = 16 * R * m;  // candidate slots: m per group
  for (int c = tid; c < C; c += kThreads) {
    cand_h[c] = kMax;
    cand_l[c] = kMax;
  }
  __syncthreads();
  // (1) rank within the group
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (hi[r] == kMax && lo[r] == kMax) continue;
    const int g0 = r * kThreads + wave * 64;
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < 64; ++q) {
      const u64x2 kq = kpair[g0 + q];
      rank += key_less(kq.x, kq.y, hi[r], lo[r]);
    }
    if (rank < m) {
      const int c = (r * 16 + wave) * m + rank;
      cand_h[c] = hi[r];
      cand_l[c] = lo[r];
    }
  }
  __syncthreads();
  // (2) rank among the candidates, split over `parts` threads per candidate
  const int parts = kThreads / C;
  for (int slot = tid; slot < C * parts; slot += kThreads) {
    const int c = slot % C, part = slot / C;
    const uint64_t ch = cand_h[c], cl = cand_l[c];
    const int q0 = C * part / parts, q1 = C * (part + 1) / parts;
    int n = 0;
    for (int q = q0; q < q1; ++q) n += key_less(cand_h[q], cand_l[q], ch, cl);
    cnt[slot] = n;
  }
  __syncthreads();
  for (int c = tid; c < C; c += kThreads) {
    const uint64_t ch = cand_h[c], cl = cand_l[c];
    if (ch == kMax && cl == kMax) continue;
    int rank = 0;
    for (int part = 0; part < parts; ++part) rank += cnt[part * C + c];
    if (rank < m) {
      khi[rank] = ch;
      klo[rank] = cl;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void lru_remap_kernel(LruArgs a) {
  // victim keys: khi / klo (sort) or interleaved pairs over the same bytes (ranks)
  __shared__ __align__(16) uint64_t kbuf[2 * OES_MAX_SLOTS];
  uint64_t *khi = kbuf, *klo = kbuf + OES_MAX_SLOTS;
  u64x2 *kpair = reinterpret_cast<u64x2 *>(kbuf);
  __shared__ int32_t emap[OES_MAX_EXPERTS];
  __shared__ int32_t mrank[OES_MAX_EXPERTS];
  __shared__ uint8_t req[OES_MAX_EXPERTS];
  __shared__ int wave_tot[kWaves + 1];
  __shared__ uint64_t cand_h[kRankCand], cand_l[kRankCand];
  __shared__ int cnt[kThreads];
  __shared__ int s_bad, s_evict;
  __shared__ uint64_t s_clock;

  const int tid = threadIdx.x;
  const int E = a.E, S = a.S;
  const int64_t base = (int64_t)a.layer * E;

  for (int e = tid; e < E; e += kThreads) {
    req[e] = 0;
    emap[e] = -1;
  }
  if (tid == 0) {
    s_bad = 0;
    s_evict = 0;
    s_clock = a.ctl->clock;
  }
  __syncthreads();

  // 1. mark requested experts, validate ids
  for (int i = tid; i < a.nk; i += kThreads) {
    const int id = a.ids[i];
    if (id < 0 || id >= E)
      s_bad = 1;
    else
      req[id] = 1;
  }
  // 2. experts of this layer that already own a slot
  for (int s = tid; s < S; s += kThreads) {
    const int64_t o = a.owner[s];
    if (o >= base && o < base + E) emap[(int)(o - base)] = s;
  }
  __syncthreads();

  // 3. misses: requested experts without a slot, ranked in ascending expert order
  int cnt_req = 0, cnt_miss = 0;
  const int e0 = tid * kPerThread;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = e0 + q;
    if (e < E && req[e]) {
      ++cnt_req;
      if (emap[e] < 0) ++cnt_miss;
    }
  }
  int nU = 0, nM = 0;
  (void)block_exclusive_scan(cnt_req, wave_tot, &nU);
  int mbase = block_exclusive_scan(cnt_miss, wave_tot, &nM);
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = e0 + q;
    if (e < E) {
      const bool m = req[e] && emap[e] < 0;
      mrank[e] = m ? mbase : -1;
      if (m) ++mbase;
    }
  }

  const bool bad = s_bad != 0;
  const bool over = !a.hybrid && nU > S;
  if (bad || over) {
    for (int i = tid; i < a.nk; i += kThreads) a.slot_ids[i] = -1;
    if (tid == 0) {
      if (a.ctl->err == OES_OK) a.ctl->err = bad ? OES_ERR_ARG : OES_ERR_CAPACITY;
      a.ctl->step_ok = 0;
      a.ctl->miss_count = 0;
      a.ctl->failed_steps += 1;
    }
    return;
  }

  // misses installed this step: all of them, or the hybrid cap
  int take = nM;
  if (a.hybrid) {
    long long cap;
    if (a.max_fetch >= 0)
      cap = a.max_fetch;
    else if (a.fetch_fraction >= 0.0)
      cap = (long long)rint((double)nM * fmin(1.0, a.fetch_fraction));
    else
      cap = 1;
    const long long avail = (long long)S - (nU - nM);  // slots not holding a member of U
    take = (int)min(cap, min((long long)nM, avail));
  }
  if (take > 0) {
    // 4-5. victim keys ascending (slots holding a member of U sort last): the
    // first `take` of them, by ranks when the candidates fit, else by a full sort
    const int R = a.Spad <= kThreads ? 1 : (a.Spad <= 2 * kThreads ? 2 : 4);
    if (16 * R * take <= kRankCand) {
      if (R == 1)
        rank_victims<1>(a, req, base, take, khi, klo, kpair, cand_h, cand_l, cnt);
      else if (R == 2)
        rank_victims<2>(a, req, base, take, khi, klo, kpair, cand_h, cand_l, cnt);
      else
        rank_victims<4>(a, req, base, take, khi, klo, kpair, cand_h, cand_l, cnt);
    } else if (a.Spad <= kThreads) {
      sort_victims<1>(a, req, base, khi, klo);
    } else if (a.Spad <= 2 * kThreads) {
      sort_victims<2>(a, req, base, khi, klo);
    } else {
      sort_victims<4>(a, req, base, khi, klo);
    }
    // 6. install: the i-th miss takes the i-th victim (hybrid: the first `take` misses)
    for (int e = tid; e < E; e += kThreads) {
      const int r = mrank[e];
      if (r >= 0 && r < take) {
        const int v = (int)(klo[r] & 0xFFFull);
        const int64_t old = a.owner[v];
        if (old != -1) atomicAdd(&s_evict, 1);
        a.owner[v] = base + e;
        emap[e] = v;
        a.miss_slot[r] = v;
        a.miss_id[r] = base + e;
      }
    }
  }
  __syncthreads();

  // 7. stamp every slot holding a member of U, then the slot map (hybrid: ids
  // left without a slot are not stamped and their requests map to -1)
  const uint64_t T = s_clock + 1;
  for (int e = tid; e < E; e += kThreads)
    if (req[e] && emap[e] >= 0) a.stamp[emap[e]] = T;
  for (int i = tid; i < a.nk; i += kThreads) a.slot_ids[i] = emap[a.ids[i]];
  if (tid == 0) {
    Ctl *c = a.ctl;
    c->clock = T;
    c->step_ok = 1;
    c->miss_count = take;
    c->steps += 1;
    c->hits += (uint64_t)(nU - nM);
    c->misses += (uint64_t)take;
    c->evictions += (uint64_t)s_evict;
    c->bytes += (uint64_t)take * (uint64_t)a.bpe;
    c->last_misses = (uint32_t)take;
    c->last_indices = (uint32_t)take;
    c->last_missing_full = (uint32_t)nM;
    c->cpu_experts += (uint64_t)(nM - take);
  }
}

__global__ void reset_step_kernel(Ctl *ctl) {
  ctl->step_ok = 1;
  ctl->miss_count = 0;
}

}  // namespace

void launch_reset_step(Ctl *ctl, hipStream_t s) { hipLaunchKernelGGL(reset_step_kernel, dim3(1), dim3(1), 0, s, ctl); }

hipError_t launch_lru_remap(const LruArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(lru_remap_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace oes
