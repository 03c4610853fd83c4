// Top-k routing: router logits x . Wg, softmax, top-k, renormalised weights.
//
// The pages name the top-k of each MoE layer (FreeToken MoE benchmark guide §4.3
// routes bs * topk experts per step) but not the router; this is the plain one.
//
// Two launches, each one memory round trip deep (one for small routers, below):
//   route_partial  - split-K GEMV: workgroup s sums rows [s*R, (s+1)*R) of
//                    Wg [H, E] (bf16, row-major) against every token, fp32,
//                    writing partial[s][t][e]; each thread owns one column octet
//                    (a 16-byte load per row, coalesced along E) and up to 16
//                    rows whose loads are all issued before the first multiply.
//   route_finish   - one workgroup per token: all threads sum the partials
//                    (deterministic order) and write the logits; each expert's
//                    rank (experts with a larger logit, or an equal one at a
//                    lower index) picks the top-k in order; one wave takes the
//                    softmax over the chosen logits.
// route_logits runs route_finish alone on given logits (one split).  When Wg fits
// one split (small routers), route_single does both in one launch: one workgroup
// per token computes its logits and takes the top-k.

#include <math.h>

#include <algorithm>

#include "oes_internal.h"

namespace oes {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRpt = 16;        // rows per thread, all loads issued at once
constexpr int kMaxTok = 32;     // tokens per pass of the partial kernel

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

struct RouteGeom {
  int cpt;    // column octets per row (E / 8)
  int rpp;    // rows processed in parallel by a workgroup
  int rows;   // rows per split (rpp * rows per thread)
  int splits;
};

RouteGeom route_geom(int H, int E) {
  RouteGeom g;
  g.cpt = E / 8;
  g.rpp = std::max(1, kRouteThreads / g.cpt);
  // rows per thread: at most kRpt, and at most 256 rows per split (the x tile in LDS)
  const int rpt = std::max(1, std::min(std::min(kRpt, 256 / g.rpp), (H + g.rpp - 1) / g.rpp));
  g.rows = g.rpp * rpt;
  g.splits = (H + g.rows - 1) / g.rows;
  return g;
}

// Split-K GEMV: workgroup s owns rows [s*rows, (s+1)*rows) of Wg [H, E].  Thread
// (sub, co) owns column octet co (one 16-byte load per row) and rows sub, sub +
// rpp, ...; it issues every row load before the first multiply.  The x values
// of the workgroup's rows are staged in LDS once.
__global__ __launch_bounds__(kRouteThreads) void route_partial_kernel(const uint16_t *x, const uint16_t *wg, int n,
                                                                      int H, int E, RouteGeom geo, float *partial) {
  __shared__ float xs[kMaxTok * 256];    // [tok][row-in-split], rows <= 256
  __shared__ float red[kRouteThreads * 8];
  const int cpt = geo.cpt, rpp = geo.rpp;
  const int sub = threadIdx.x / cpt, co = threadIdx.x % cpt;
  const bool active = sub < rpp;
  const int r0 = blockIdx.x * geo.rows;
  const int nrows = min(geo.rows, H - r0);
  u32x4 wv[kRpt];
#pragma unroll
  for (int i = 0; i < kRpt; ++i) {
    const int rl = sub + i * rpp;
    if (active && rl < nrows) wv[i] = *reinterpret_cast<const u32x4 *>(wg + (int64_t)(r0 + rl) * E + co * 8);
  }
  for (int t0 = 0; t0 < n; t0 += kMaxTok) {
    const int tn = min(kMaxTok, n - t0);
    __syncthreads();
    for (int i = threadIdx.x; i < tn * nrows; i += kRouteThreads) {
      const int t = i / nrows, rl = i % nrows;
      xs[t * 256 + rl] = bf16f(x[(int64_t)(t0 + t) * H + r0 + rl]);
    }
    __syncthreads();
    for (int t = 0; t < tn; ++t) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (active) {
#pragma unroll
        for (int i = 0; i < kRpt; ++i) {
          const int rl = sub + i * rpp;
          if (rl < nrows) {
            const float xv = xs[t * 256 + rl];
            const u32x4 w = wv[i];
            acc[0] = fmaf(xv, __uint_as_float(w.x << 16), acc[0]);
            acc[1] = fmaf(xv, __uint_as_float(w.x & 0xffff0000u), acc[1]);
            acc[2] = fmaf(xv, __uint_as_float(w.y << 16), acc[2]);
            acc[3] = fmaf(xv, __uint_as_float(w.y & 0xffff0000u), acc[3]);
            acc[4] = fmaf(xv, __uint_as_float(w.z << 16), acc[4]);
            acc[5] = fmaf(xv, __uint_as_float(w.z & 0xffff0000u), acc[5]);
            acc[6] = fmaf(xv, __uint_as_float(w.w << 16), acc[6]);
            acc[7] = fmaf(xv, __uint_as_float(w.w & 0xffff0000u), acc[7]);
          }
        }
      }
      // reduce the rpp row groups through LDS, in fixed order
      if (active)
#pragma unroll
        for (int c = 0; c < 8; ++c) red[sub * E + co * 8 + c] = acc[c];
      __syncthreads();
      for (int e = threadIdx.x; e < E; e += kRouteThreads) {
        float s = 0.f;
        for (int g = 0; g < rpp; ++g) s += red[g * E + e];
        partial[((int64_t)blockIdx.x * n + t0 + t) * E + e] = s;
      }
      __syncthreads();
    }
  }
}

// One workgroup per token.  All 256 threads sum the split partials (thread i
// takes expert i % E and splits i / E, i / E + 256 / E, ... with independent
// loads; the per-thread sums are added in a fixed order through LDS, so the
// result is deterministic).  Then the top-k by rank (larger logit first, lower
// index on ties); lane j of wave 0 takes the j-th pick and writes its id and
// renormalised weight.
struct FinishSmem {
  float zsum[kRouteThreads];
  float z[512];
  float top_v[32];
  int top_i[32];
  __align__(16) uint64_t rkey[512 + 2];
  int rcnt[512];
};

__device__ __forceinline__ void finish_topk(FinishSmem &sm, int t, int E, int k, int32_t *ids, float *w);

__global__ __launch_bounds__(kRouteThreads) void route_finish_kernel(const float *partial, int splits, int n, int E,
                                                                     int k, float *logits, int32_t *ids, float *w) {
  __shared__ FinishSmem sm;
  float *zsum = sm.zsum, *z = sm.z;
  const int t = blockIdx.x;
  const int64_t stride = (int64_t)n * E;
  const int per = kRouteThreads / E >= 1 ? kRouteThreads / E : 1;   // threads per expert (E <= 256)
  if (E <= kRouteThreads) {
    const int e = threadIdx.x % E, part = threadIdx.x / E;
    float s = 0.f;
    if (part < per) {
      const float *p = partial + (int64_t)t * E + e;
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
      int sp = part;
      for (; sp + 3 * per < splits; sp += 4 * per) {
        a4[0] += p[(sp + 0 * per) * stride];
        a4[1] += p[(sp + 1 * per) * stride];
        a4[2] += p[(sp + 2 * per) * stride];
        a4[3] += p[(sp + 3 * per) * stride];
      }
      for (; sp < splits; sp += per) a4[0] += p[sp * stride];
      s = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    }
    zsum[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x < E) {
      float tot = 0.f;
      for (int q = 0; q < per; ++q) tot += zsum[q * E + threadIdx.x];
      z[threadIdx.x] = tot;
      if (logits) logits[(int64_t)t * E + threadIdx.x] = tot;
    }
  } else {
    for (int e = threadIdx.x; e < E; e += kRouteThreads) {
      const float *p = partial + (int64_t)t * E + e;
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
      int sp = 0;
      for (; sp + 4 <= splits; sp += 4) {
        a4[0] += p[(sp + 0) * stride];
        a4[1] += p[(sp + 1) * stride];
        a4[2] += p[(sp + 2) * stride];
        a4[3] += p[(sp + 3) * stride];
      }
      for (; sp < splits; ++sp) a4[0] += p[sp * stride];
      const float tot = (a4[0] + a4[1]) + (a4[2] + a4[3]);
      z[e] = tot;
      if (logits) logits[(int64_t)t * E + e] = tot;
    }
  }
  __syncthreads();
  finish_topk(sm, t, E, k, ids, w);
}

// The top-k of the logits sm.z[0, E) of token t (all threads of the workgroup;
// sm.z written and synchronised by the caller).
__device__ __forceinline__ void finish_topk(FinishSmem &sm, int t, int E, int k, int32_t *ids, float *w) {
  float *z = sm.z, *top_v = sm.top_v;
  int *top_i = sm.top_i, *rcnt = sm.rcnt;
  uint64_t *rkey = sm.rkey;
  // top-k by rank: expert e's rank is the number of experts that beat it - a larger
  // logit, or an equal one at a lower index; a NaN logit is beaten by every number
  // and NaNs among themselves go by index.  Each expert gets one 64-bit key that
  // orders exactly so (the logit mapped to an order-preserving integer, -0 as +0
  // and NaN below -inf, then the inverted index), so the ranks are a permutation
  // and rank(e) = #{q : key[q] > key[e]}; the k experts of rank < k are the
  // picks, in order.  Each expert's count is split over up to 256 / E threads
  // that read two keys per 16-byte LDS load.
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    float v = z[e];
    if (v == 0.f) v = 0.f;
    const uint32_t u = __float_as_uint(v);
    const uint32_t ord = v != v ? 0u : ((u >> 31) ? ~u : (u | 0x80000000u));
    rkey[e] = ((uint64_t)ord << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
  }
  if ((E & 1) && threadIdx.x == 0) rkey[E] = 0;  // pad to an even count: beats nothing
  __syncthreads();
  {
    const int parts = E <= kRouteThreads / 2 ? kRouteThreads / E : 1;
    const int E2 = (E + 1) / 2;                        // key pairs
    for (int slot = threadIdx.x; slot < E * parts; slot += kRouteThreads) {
      const int e = slot % E, part = slot / E;
      const uint64_t ke = rkey[e];
      const int q0 = E2 * part / parts, q1 = E2 * (part + 1) / parts;
      const u64x2 *kp = reinterpret_cast<const u64x2 *>(rkey);
      int cnt = 0;
#pragma unroll 8
      for (int q = q0; q < q1; ++q) {
        const u64x2 kk = kp[q];
        cnt += (kk.x > ke) + (kk.y > ke);
      }
      rcnt[slot] = cnt;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    const int parts = E <= kRouteThreads / 2 ? kRouteThreads / E : 1;
    int rank = 0;
    for (int part = 0; part < parts; ++part) rank += rcnt[part * E + e];
    if (rank < k) {
      top_v[rank] = z[e];
      top_i[rank] = e;
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const float myv = lane < k ? top_v[lane] : 0.f;
  const int myi = lane < k ? top_i[lane] : 0;
  const float v0 = __shfl(myv, 0, 64);
  const float ex = lane < k ? expf(myv - v0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) sum += __shfl_xor(sum, d, 64);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = myi;
    w[(int64_t)t * k + lane] = ex / sum;
  }
}

// Routing in one launch when Wg fits one split (H <= the rows of a split, as for
// small routers): one workgroup per token computes its logits and takes the top-k.
// Thread (part, e) sums rows part, part + parts, ... of column e in fp32; the parts
// are added in a fixed order through LDS.
__global__ __launch_bounds__(kRouteThreads) void route_single_kernel(const uint16_t *x, const uint16_t *wg, int H,
                                                                     int E, int k, float *logits, int32_t *ids,
                                                                     float *w) {
  __shared__ FinishSmem sm;
  const int t = blockIdx.x;
  const int parts = kRouteThreads / E;  // E <= 256
  const int e = threadIdx.x % E, part = threadIdx.x / E;
  float s = 0.f;
  if (part < parts)
    for (int h = part; h < H; h += parts) s = fmaf(bf16f(x[(int64_t)t * H + h]), bf16f(wg[(int64_t)h * E + e]), s);
  sm.zsum[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < E) {
    float tot = 0.f;
    for (int q = 0; q < parts; ++q) tot += sm.zsum[q * E + threadIdx.x];
    sm.z[threadIdx.x] = tot;
    if (logits) logits[(int64_t)t * E + threadIdx.x] = tot;
  }
  __syncthreads();
  finish_topk(sm, t, E, k, ids, w);
}

}  // namespace

int route_splits(int H, int E) { return route_geom(H, E).splits; }

hipError_t launch_route(const uint16_t *x, const uint16_t *wg, int n, int H, int E, int k, int32_t *ids, float *w,
                        float *logits, float *partial, hipStream_t s) {
  const RouteGeom geo = route_geom(H, E);
  if (geo.splits == 1 && E <= kRouteThreads) {
    hipLaunchKernelGGL(route_single_kernel, dim3(n), dim3(kRouteThreads), 0, s, x, wg, H, E, k, logits, ids, w);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_partial_kernel, dim3(geo.splits), dim3(kRouteThreads), 0, s, x, wg, n, H, E, geo, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_finish_kernel, dim3(n), dim3(kRouteThreads), 0, s, partial, geo.splits, n, E, k, logits,
                     ids, w);
  return hipGetLastError();
}

hipError_t launch_route_logits(const float *logits, int n, int E, int k, int32_t *ids, float *w, hipStream_t s) {
  hipLaunchKernelGGL(route_finish_kernel, dim3(n), dim3(kRouteThreads), 0, s, logits, 1, n, E, k,
                     static_cast<float *>(nullptr), ids, w);
  return hipGetLastError();
}

}  // namespace oes
