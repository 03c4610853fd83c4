// Prefill grouped expert FFN over a streamed layer buffer: MXFP4 weights, bf16 MFMA.
//
// FreeToken architecture walk-through §5: prefill streams whole layers through a
// double buffer; the FFN of a layer runs on the buffer holding it (row e =
// expert e).  FreeToken MoE benchmark guide §4.2: the MXFP4 format keeps six
// transposed banks - _blocks, _scales, _bias for gate_up and for down.
//
// Four launches:
//   permute    - one workgroup counts the (token, pair) routes per expert, scans
//                the counts into offsets and scatters the pair indices into
//                expert order (perm).  The order inside an expert does not
//                change any result: every output row of a GEMM is computed on
//                its own, with the same k order.
//   gemm<0>    - per expert e: h = silu(X_e Wg_e^T + bg) * (X_e Wu_e^T + bu), bf16,
//                X_e the gathered activation rows of the pairs routed to e.
//   gemm<1>    - per expert e: o = h_e Wd_e^T + bd, fp32, scattered back to the
//                pair's row.
//   combine    - y_t = sum_j w[t, j] * o_{t,j} in pair order, bf16.
//
// GEMM tiling (v_mfma_f32_32x32x16_bf16, details at the kernel):
//   block = (expert, 128 / 256 output features) x all rows of the expert in
//   passes of 96; in gate_up, wave w owns 32 features (those 32 gate rows and
//   the matching 32 up rows, so silu(g) * u is formed in registers).  K runs in
//   quads of four 32-element MXFP4 blocks.  The A chunk of a quad is staged in
//   LDS from registers loaded one quad ahead; the B operand needs no LDS: the
//   K-block-major layout [K/32][N][16 B] gives each lane one 16-byte load per
//   pair of blocks that feeds four MFMAs after fp4 -> bf16 scaled conversions
//   (exact: e2m1 * 2^k is a bf16 number).
//   Blocks are mapped XCD-aware: hardware deals consecutive block indices to
//   the 8 XCDs in turn, so block b runs on XCD b % 8; experts e with e % 8 == x
//   are given to XCD x, which keeps an expert's activation rows in one L2
//   while all its feature tiles stream their weights.

#include <math.h>

#include <algorithm>

#include "oes_internal.h"

namespace oes {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;  // a global-memory u32x4

constexpr int kThreads = 256;
constexpr int BM = 96;             // rows per pass: three 32-row m-tiles
constexpr int LDA = 128 + 8;       // LDS row of one 128-k quad, bf16 elements, padded 16 B
constexpr int kXcds = 8;
constexpr int kProbeChains = 4;    // accumulator chains per wave of the MFMA ceiling probe
constexpr int kMaxKb = 96;         // K / 32 limit of the grouped GEMM (K <= 3072)
static_assert(kThreads == 256, "two A pieces per thread cover one row of each half m-tile");

struct GemmArgs {
  int32_t H, I, E, k, nk;
  int32_t ntiles;        // feature tiles per expert
  int32_t xcd;           // 1: XCD-aware block mapping (E % 8 == 0)
  const uint16_t *x;     // [n, H] bf16
  const int32_t *offsets;  // [E + 1]
  const int32_t *perm;     // [nk] pair indices in expert order
  const uint8_t *blocks;   // this phase's _blocks bank, expert stride blocks_stride
  const uint8_t *scales;   // this phase's _scales bank
  const uint16_t *bias;    // this phase's _bias bank (bf16)
  int64_t blocks_stride, scales_stride, bias_stride;
  const u32x4 *zero16;   // 16 zero bytes: the source of A pieces past K
  uint16_t *hbuf;        // [nk, I] bf16, expert order
  float *obuf;           // [nk, H] fp32, pair order
};

__device__ inline float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ inline uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// e8m0 byte -> fp32 scale 2^(e-127); 0 -> 2^-127 (subnormal), 255 -> NaN
__device__ inline float e8m0f(uint32_t e) {
  return e == 255u ? __uint_as_float(0x7fc00000u) : (e == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23));
}
// eight e2m1 codes (low nibble first) times a power-of-two scale -> bf16x8 operand
__device__ inline bf16x8 fp4x8_bf16(uint32_t v, float s) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// ------------------------------------------------------------------ permute
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t *ids, int nk, int E, int32_t *offsets,
                                                       int32_t *perm, uint32_t *zeros) {
  if (threadIdx.x < 64) zeros[threadIdx.x] = 0u;  // the GEMMs' 256-byte zero source
  __shared__ int hist[OES_MAX_EXPERTS];
  __shared__ int cursor[OES_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < nk; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      cursor[e] = run;
      offsets[e] = run;
      run += hist[e];
    }
    offsets[E] = run;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < nk; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) perm[atomicAdd(&cursor[e], 1)] = p;
  }
}

// ------------------------------------------------------------------ grouped GEMM
// Block = (expert, feature tile), 4 waves; rows of the expert in passes of at
// most BM = 96, each pass run by a body specialised on its count of 32-row
// m-tiles so that its quad loop has no branches.  v_mfma_f32_32x32x16_bf16:
// lane l holds A[l%32][8(l/32)..+7] and B[8(l/32)..+7][l%32]; D element r of
// lane l is row 4(l/32) + (r%4) + 8(r/4), column l%32.
//
// K order.  K runs in quads of four 32-element MXFP4 blocks (128 k), a quad in
// two pairs.  An MFMA sums over its 16 k-slots in any order as long as A and B
// use the same one, so in step j (0..3) of the pair starting at block kb0, lane
// half h = l/32 feeds k-slots 8h..8h+7 with the real k = 32(kb0 + h) + 8j + i.
// Lane (n, h) then needs all 32 codes of block kb0 + h of weight row n: the 16
// contiguous bytes at (kb0 + h, n) of the [K/32][N][16] bank, one 16-byte load
// per lane for four MFMAs, with one scale byte.
//
// Pipelining.  The block's scale bytes (its 256 weight rows x K/32 blocks) are
// copied to LDS once.  B: each wave holds one quad's two pairs per n-tile in
// registers; pair p of quad q + 1 is loaded as soon as quad q's MFMA steps on
// pair p are issued.  A: the chunk of quad q + 1 (the pass's rows x 128 k,
// bf16) is loaded into registers while quad q is multiplied from LDS, then
// stored to the other LDS buffer; one barrier per quad.  The steady-state loop
// has no conditions, so the compiler's memory-counter waits stay exact.
// Indexes past the data are clamped (B) or pointed at a zero block (A, k past
// K), never branched on.  Each output row of an MFMA depends only on its own A
// row, so A rows past the pass's last row may hold anything: their outputs are
// never stored.
//
// Each wave owns two 32-feature n-tiles: gate_up - the gate tile and the up
// tile of the same 32 features (128 features per block); down - two consecutive
// tiles (256 features per block).  Tiles past the last feature run on clamped
// rows and are not stored.
constexpr int kUnroll = 2;  // quads per steady-state iteration: the LDS buffer parity is static
constexpr int NTW = 2;
constexpr int kRowsB = 256;  // weight rows per block

struct Tile {
  int e, off, m0, mrows;
  int K, N, nkb, nq;
  int nrow[NTW], f[NTW], lrow[NTW];
  bool tile_on[NTW];
  int n32, h;
};

// e8m0 byte -> fp32 2^(e-127): e << 23, with 0 -> 2^-127 (0x00400000) and
// 255 -> NaN (0x7fc00000), both by setting bit 22; no branches
__device__ __forceinline__ float e8m0_bits(uint32_t e) {
  return __uint_as_float((e << 23) | ((uint32_t)(e == 0u || e == 255u) << 22));
}

template <int PHASE, int MT>
__device__ __forceinline__ void gemm_pass(const GemmArgs &g, const Tile &T, uint16_t (*As)[BM * LDA],
                                          const int32_t *rowoff, const uint8_t *sc_lds) {
  constexpr int AP = 2 * MT;  // 16-byte A pieces per thread per quad
  const uint8_t *blk = g.blocks + (int64_t)T.e * g.blocks_stride;
  const uint16_t *asrc = PHASE == 0 ? g.x : g.hbuf;
  const int n32 = T.n32, h = T.h;
  const int c16 = threadIdx.x & 15, rsub = threadIdx.x >> 4;  // A piece: row 16i + rsub, column c16

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  // A rows: rowoff < 0 marks a row past the pass (read row 0 instead)
  int32_t aoff[AP];
#pragma unroll
  for (int i = 0; i < AP; ++i) aoff[i] = max(rowoff[16 * i + rsub], 0);
  // pieces past K read the zero block: a select on the loaded value would make
  // the wave wait for the loads at once instead of at the quad's end
  const uint64_t zero_addr = reinterpret_cast<uint64_t>(g.zero16);
  u32x4 areg[AP];
  auto load_a = [&](int q) {
    const int k0 = q * 128 + c16 * 8;
    const bool kin = k0 < T.K;
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      uint64_t src = kin ? reinterpret_cast<uint64_t>(asrc + aoff[i] + k0) : zero_addr;
      asm volatile("" : "+v"(src));  // keep the select on the address
      areg[i] = __builtin_nontemporal_load(reinterpret_cast<const gu32x4 *>(src));
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AP; ++i) *reinterpret_cast<u32x4 *>(&As[buf][(16 * i + rsub) * LDA + c16 * 8]) = areg[i];
  };
  // B: one quad's two pairs; pair p of quad q + 1 is loaded as soon as quad q's
  // steps on pair p are issued
  u32x4 bw[2][NTW];
  const int64_t kstride = (int64_t)T.N * 16;
  uint32_t boff[NTW], soff[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    boff[t] = (uint32_t)(T.nrow[t] * 16 + h * T.N * 16);
    soff[t] = (uint32_t)(h * kRowsB + T.lrow[t]);
  }
  auto pair_kb0 = [&](int p, int q) { return min(4 * q + 2 * p, T.nkb - 2); };
  auto load_bp = [&](int p, int q) {
    const uint8_t *ub = blk + (int64_t)pair_kb0(p, q) * kstride;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      bw[p][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ub + boff[t]));
  };

  auto quad = [&](int q, bool more) {
    if (more) load_a(q + 1);
    const uint16_t *Ab = As[q & 1];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint8_t *sl = sc_lds + pair_kb0(p, q) * kRowsB;
      float sc[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) sc[t] = e8m0_bits(sl[soff[t]]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 bop[NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t) bop[t] = fp4x8_bf16(bw[p][t][j], sc[t]);
        if (j == 3) load_bp(p, q + 1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 av =
              *reinterpret_cast<const bf16x8 *>(&Ab[(mt * 32 + n32) * LDA + (2 * p + h) * 32 + j * 8]);
#pragma unroll
          for (int t = 0; t < NTW; ++t)
            acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bop[t], acc[mt][t], 0, 0, 0);
        }
      }
    }
    if (more) store_a((q + 1) & 1);
    __syncthreads();
  };

  load_bp(0, 0);
  load_bp(1, 0);
  load_a(0);
  store_a(0);
  __syncthreads();
  // steady state: every quad of the group has a successor
  int q0 = 0;
  for (; q0 + kUnroll < T.nq; q0 += kUnroll) {
#pragma unroll
    for (int d = 0; d < kUnroll; ++d) quad(q0 + d, true);
  }
  // the last one to kUnroll quads
#pragma unroll
  for (int d = 0; d < kUnroll; ++d)
    if (q0 + d < T.nq) quad(q0 + d, q0 + d + 1 < T.nq);

  // epilogue: acc[mt][t][r] is row mt*32 + 4h + (r%4) + 8(r/4) of the pass, feature f[t]
  const uint16_t *bias = g.bias + (int64_t)T.e * g.bias_stride;
  if (PHASE == 0) {
    if (T.tile_on[0]) {
      const float bg = bf16f(bias[T.f[0]]), bu = bf16f(bias[g.I + T.f[0]]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mt * 32 + 4 * h + (r & 3) + 8 * (r >> 2);
          if (m < T.mrows) {
            const float gv = acc[mt][0][r] + bg, uv = acc[mt][1][r] + bu;
            const float hv = gv / (1.f + __expf(-gv)) * uv;
            g.hbuf[(int64_t)(T.off + T.m0 + m) * g.I + T.f[0]] = to_bf16(hv);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      if (!T.tile_on[t]) continue;
      const float bd = bf16f(bias[T.f[t]]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mt * 32 + 4 * h + (r & 3) + 8 * (r >> 2);
          if (m < T.mrows) {
            const int pr = g.perm[T.off + T.m0 + m];
            g.obuf[(int64_t)pr * g.H + T.f[t]] = acc[mt][t][r] + bd;
          }
        }
      }
    }
  }
}

template <int PHASE>
__global__ __launch_bounds__(kThreads, 2) void moe_gemm_kernel(GemmArgs g) {
  constexpr int NFB = PHASE == 0 ? 128 : 256;  // features per block
  __shared__ __align__(16) uint16_t As[2][BM * LDA];
  __shared__ int32_t rowoff[BM];
  __shared__ __align__(16) uint8_t sc_lds[kMaxKb * kRowsB];
  Tile T;
  int nt;
  if (g.xcd) {
    const int x = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
    T.e = x + kXcds * (local / g.ntiles);
    nt = local % g.ntiles;
  } else {
    T.e = blockIdx.x / g.ntiles;
    nt = blockIdx.x % g.ntiles;
  }
  if (T.e >= g.E) return;
  T.off = g.offsets[T.e];
  const int m_e = g.offsets[T.e + 1] - T.off;
  if (m_e <= 0) return;
  T.K = PHASE == 0 ? g.H : g.I;
  T.N = PHASE == 0 ? 2 * g.I : g.H;
  const int nfeat = PHASE == 0 ? g.I : g.H;
  T.nkb = T.K / 32;
  T.nq = (T.nkb + 3) >> 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  T.n32 = lane & 31;
  T.h = lane >> 5;
  if (PHASE == 0) {
    const int fbase = nt * NFB + wave * 32;
    T.f[0] = T.f[1] = fbase + T.n32;
    T.nrow[0] = min(T.f[0], g.I - 1);
    T.nrow[1] = g.I + T.nrow[0];
    T.lrow[0] = wave * 32 + T.n32;
    T.lrow[1] = 128 + T.lrow[0];
    T.tile_on[0] = T.tile_on[1] = fbase < nfeat;
  } else {
    const int fbase = nt * NFB + wave * 64;
    T.f[0] = fbase + T.n32;
    T.f[1] = T.f[0] + 32;
    T.nrow[0] = min(T.f[0], T.N - 1);
    T.nrow[1] = min(T.f[1], T.N - 1);
    T.lrow[0] = wave * 64 + T.n32;
    T.lrow[1] = T.lrow[0] + 32;
    T.tile_on[0] = fbase < nfeat;
    T.tile_on[1] = fbase + 32 < nfeat;
  }
  // scale bytes of the block's 256 weight rows: sc_lds[kb][local row], taken as
  // dwords of four rows (rows past the matrix clamp to its last dword; their
  // tiles are never stored).  Thread (w, c) copies dword c of blocks w, w + 4,
  // ..., w + 92: every load is issued before the first LDS write, so the staging
  // costs one memory round trip instead of one per dword.  Blocks past K / 32
  // get copies of the last block (the array holds kMaxKb of them; the quad loop
  // clamps its block index below K / 32, so they are never read).
  {
    constexpr int kScPer = kMaxKb * (kRowsB / 4) / kThreads;  // dwords per thread at most
    static_assert(kRowsB / 4 == 64 && kThreads == 256, "a wave copies one scale block row per step");
    const int r4 = lane * 4;
    int row;
    if (PHASE == 0) row = r4 < 128 ? min(nt * 128 + r4, g.I - 4) : g.I + min(nt * 128 + r4 - 128, g.I - 4);
    else row = min(nt * 256 + r4, T.N - 4);
    const uint8_t *scl = g.scales + (int64_t)T.e * g.scales_stride + row;
    uint32_t sv[kScPer];
#pragma unroll
    for (int u = 0; u < kScPer; ++u) {
      const int kb = min(wave + 4 * u, T.nkb - 1);
      sv[u] = *reinterpret_cast<const uint32_t *>(scl + (int64_t)kb * T.N);
    }
#pragma unroll
    for (int u = 0; u < kScPer; ++u) *reinterpret_cast<uint32_t *>(&sc_lds[(wave + 4 * u) * kRowsB + r4]) = sv[u];
  }
  const int lda_src = PHASE == 0 ? g.H : g.I;

  for (T.m0 = 0; T.m0 < m_e; T.m0 += BM) {
    T.mrows = min(BM, m_e - T.m0);
    __syncthreads();  // the previous pass is done with rowoff and As; sc_lds is written
    for (int r = threadIdx.x; r < BM; r += kThreads) {
      int32_t o = -1;
      if (r < T.mrows) {
        const int32_t src_row = PHASE == 0 ? g.perm[T.off + T.m0 + r] / g.k : T.off + T.m0 + r;
        o = src_row * lda_src;
      }
      rowoff[r] = o;
    }
    __syncthreads();
    switch ((T.mrows + 31) >> 5) {
      case 1: gemm_pass<PHASE, 1>(g, T, As, rowoff, sc_lds); break;
      case 2: gemm_pass<PHASE, 2>(g, T, As, rowoff, sc_lds); break;
      default: gemm_pass<PHASE, 3>(g, T, As, rowoff, sc_lds); break;
    }
  }
}

// ------------------------------------------------------------------ MFMA ceiling
// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave, the
// instruction the grouped GEMM uses; operands stay in registers.  The result is
// stored only on an impossible value, which keeps the chains live.
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = (float)(c + r);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) t += acc[c][0] + acc[c][15];
  if (t == 1234.5678f) sink[0] = t;
}

// ------------------------------------------------------------------ combine
// y[t, c..c+3] = sum_j w[t, j] * o[t*k + j, c..c+3], pairs with an invalid id skipped.
__global__ __launch_bounds__(kThreads) void combine_kernel(const float *obuf, const int32_t *ids, const float *w, int n,
                                                           int k, int H, int E, uint16_t *y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * kThreads + threadIdx.x) * 4;
  if (t >= n || c >= H) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const float wj = w[p];
    const f32x4 o = *reinterpret_cast<const f32x4 *>(obuf + (int64_t)p * H + c);
    s[0] = fmaf(wj, o[0], s[0]);
    s[1] = fmaf(wj, o[1], s[1]);
    s[2] = fmaf(wj, o[2], s[2]);
    s[3] = fmaf(wj, o[3], s[3]);
  }
  u32x2 out;
  out[0] = (uint32_t)to_bf16(s[0]) | ((uint32_t)to_bf16(s[1]) << 16);
  out[1] = (uint32_t)to_bf16(s[2]) | ((uint32_t)to_bf16(s[3]) << 16);
  *reinterpret_cast<u32x2 *>(y + (int64_t)t * H + c) = out;
}

struct WsLayout {
  int64_t offsets, zeros, perm, hbuf, obuf, total;
};

WsLayout ws_layout(int H, int I, int n, int k, int E) {
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  WsLayout L;
  const int64_t nk = (int64_t)n * k;
  L.offsets = 0;
  L.zeros = up(4ll * (E + 1));
  L.perm = L.zeros + 256;
  L.hbuf = L.perm + up(4 * nk);
  L.obuf = L.hbuf + up(2 * nk * I);
  L.total = L.obuf + up(4 * nk * H);
  return L;
}

}  // namespace

hipError_t launch_mfma_probe(int blocks, int iters, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kThreads), 0, s, iters, sink);
  return hipGetLastError();
}

int64_t mfma_probe_flops(int blocks, int iters) {
  return (int64_t)blocks * (kThreads / 64) * iters * kProbeChains * 32 * 32 * 16 * 2;
}

bool prefill_supported(int H, int I, int E) {
  return H % 64 == 0 && I % 64 == 0 && H / 32 <= kMaxKb && I / 32 <= kMaxKb && E <= OES_MAX_EXPERTS;
}

int64_t prefill_workspace_bytes(int H, int I, int n, int k, int E) { return ws_layout(H, I, n, k, E).total; }

hipError_t launch_prefill_ffn(const PrefillArgs &a, hipStream_t s) {
  if (!prefill_supported(a.H, a.I, a.E)) return hipErrorInvalidValue;
  // A element offsets of the GEMMs are 32-bit
  if ((int64_t)a.n * a.k * std::max(a.H, a.I) >= (int64_t)1 << 31) return hipErrorInvalidValue;
  const WsLayout L = ws_layout(a.H, a.I, a.n, a.k, a.E);
  if (a.ws_bytes < L.total) return hipErrorInvalidValue;
  const int nk = a.n * a.k;
  int32_t *offsets = reinterpret_cast<int32_t *>(a.ws + L.offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(a.ws + L.perm);
  uint16_t *hbuf = reinterpret_cast<uint16_t *>(a.ws + L.hbuf);
  float *obuf = reinterpret_cast<float *>(a.ws + L.obuf);
  uint32_t *zeros = reinterpret_cast<uint32_t *>(a.ws + L.zeros);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, s, a.ids, nk, a.E, offsets, perm, zeros);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemmArgs g;
  g.zero16 = reinterpret_cast<const u32x4 *>(zeros);
  g.H = a.H;
  g.I = a.I;
  g.E = a.E;
  g.k = a.k;
  g.nk = nk;
  g.xcd = (a.E % kXcds == 0) ? 1 : 0;
  g.x = a.x;
  g.offsets = offsets;
  g.perm = perm;
  g.hbuf = hbuf;
  g.obuf = obuf;
  // gate_up: banks 0..2; features I, 64 per block
  g.blocks = a.bank[0];
  g.scales = a.bank[1];
  g.bias = reinterpret_cast<const uint16_t *>(a.bank[2]);
  g.blocks_stride = a.row_bytes[0];
  g.scales_stride = a.row_bytes[1];
  g.bias_stride = a.row_bytes[2] / 2;
  g.ntiles = (a.I + 127) / 128;
  hipLaunchKernelGGL(moe_gemm_kernel<0>, dim3(a.E * g.ntiles), dim3(kThreads), 0, s, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // down: banks 3..5; features H
  g.blocks = a.bank[3];
  g.scales = a.bank[4];
  g.bias = reinterpret_cast<const uint16_t *>(a.bank[5]);
  g.blocks_stride = a.row_bytes[3];
  g.scales_stride = a.row_bytes[4];
  g.bias_stride = a.row_bytes[5] / 2;
  g.ntiles = (a.H + 255) / 256;
  hipLaunchKernelGGL(moe_gemm_kernel<1>, dim3(a.E * g.ntiles), dim3(kThreads), 0, s, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid((a.H / 4 + kThreads - 1) / kThreads, a.n);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(kThreads), 0, s, obuf, a.ids, a.w, a.n, a.k, a.H, a.E, a.y);
  return hipGetLastError();
}

}  // namespace oes
