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
// GEMM tiling (v_mfma_f32_16x16x32_bf16; lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16], D[4(l/16)+r][l%16]):
//   block = (expert, 64 / 128 output features) x all rows of the expert in
//   passes of 96; in gate_up, wave w owns 16 features (those 16 gate rows and
//   the matching 16 up rows, so silu(g) * u is formed in registers).  K runs in
//   quads of four 32-element MXFP4 blocks.  The A chunk of a quad is staged in
//   LDS from registers loaded one quad ahead; the B operand needs no LDS: the
//   K-block-major layout [K/32][N][16 B] gives each lane one 16-byte load per
//   quad that feeds four MFMAs after fp4 -> bf16 scaled conversions (exact:
//   e2m1 * 2^k is a bf16 number).
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int BM = 96;             // rows per pass: six 16-row m-tiles
constexpr int LDA = 128 + 8;       // LDS row of one 128-k quad, bf16 elements, padded 16 B
constexpr int kXcds = 8;
static_assert(kThreads == 256, "an A piece per thread covers one row of each m-tile");

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
                                                       int32_t *perm) {
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
// most BM, each pass run by a body specialised on its m-tile count so that its
// quad loop has no branches.
//
// K order inside a quad.  K runs in quads of four 32-element MXFP4 blocks (128
// k).  An MFMA sums over its 32 k-slots in any order as long as A and B use the
// same one, so in MFMA step j (0..3) of a quad starting at block kb0, lane group
// lq = l/16 feeds k-slots 8lq..8lq+7 with the real k = 32(kb0 + lq) + 8j + i.
// Lane (l16, lq) then needs all 32 codes of block kb0 + lq of its row, which are
// the 16 contiguous bytes at (kb0 + lq, row) of the [K/32][N][16] bank: one
// 16-byte load per lane feeds four MFMAs, and its one scale byte covers them.
//
// Pipelining.  B: each wave keeps a ring of KRING quads per n-tile in registers;
// the slot of quad q is converted to bf16 and at once refilled with quad
// q + KRING.  A: the chunk of quad q + 1 (16 rows per m-tile x 128 k, bf16) is
// loaded into registers while quad q is multiplied from LDS, then stored to the
// other LDS buffer; one barrier per quad.  Each output row of an MFMA depends
// only on its own A row, so A rows past the pass's last row are left as they are
// (their outputs are never stored); k past K is zero, against clamped B blocks.
//
// Each wave owns two 16-feature n-tiles: gate_up - the gate tile and the up tile
// of the same 16 features (64 features per block); down - two consecutive tiles
// (128 features per block; tiles past the last feature are computed on clamped
// rows and not stored).
constexpr int KRING = 3;
constexpr int NTW = 2;

struct Tile {
  int e, off, m0, mrows;
  int K, N, nkb, nq;
  int nrow[NTW], f[NTW];
  bool tile_on[NTW];
  int l16, lq;
};

template <int PHASE, int MTS>
__device__ __forceinline__ void gemm_pass(const GemmArgs &g, const Tile &T, uint16_t (*As)[BM * LDA],
                                          const int64_t *rowoff) {
  const uint8_t *blk = g.blocks + (int64_t)T.e * g.blocks_stride;
  const uint8_t *scl = g.scales + (int64_t)T.e * g.scales_stride;
  const uint16_t *asrc = PHASE == 0 ? g.x : g.hbuf;
  const int l16 = T.l16, lq = T.lq;
  const int c16 = threadIdx.x & 15, rsub = threadIdx.x >> 4;  // A piece: row rsub of each m-tile

  f32x4 acc[MTS][NTW];
#pragma unroll
  for (int i = 0; i < MTS; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  int64_t aoff[MTS];
#pragma unroll
  for (int i = 0; i < MTS; ++i) aoff[i] = rowoff[16 * i + rsub];
  u32x4 areg[MTS];
  auto load_a = [&](int q) {
    const int k0 = q * 128 + c16 * 8;
#pragma unroll
    for (int i = 0; i < MTS; ++i)
      areg[i] = (aoff[i] >= 0 && k0 < T.K)
                    ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(asrc + aoff[i] + k0))
                    : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MTS; ++i) *reinterpret_cast<u32x4 *>(&As[buf][(16 * i + rsub) * LDA + c16 * 8]) = areg[i];
  };
  // B ring: slot d holds quad q (q % KRING == d) for both n-tiles.  Blocks past
  // K are clamped to the last one: the A k-slots they meet are zero.
  u32x4 bw[KRING][NTW];
  uint32_t bs[KRING][NTW];
  auto load_b = [&](int d, int q) {
    const int kb = min(4 * q + lq, T.nkb - 1);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int64_t idx = (int64_t)kb * T.N + T.nrow[t];
      bw[d][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(blk + idx * 16));
      bs[d][t] = scl[idx];
    }
  };

#pragma unroll
  for (int d = 0; d < KRING; ++d) load_b(d, d);
  load_a(0);
  store_a(0);
  __syncthreads();
  for (int q0 = 0; q0 < T.nq; q0 += KRING) {
#pragma unroll
    for (int d = 0; d < KRING; ++d) {
      const int q = q0 + d;
      if (q < T.nq) {
        const bool more = q + 1 < T.nq;
        if (more) load_a(q + 1);
        bf16x8 bop[4][NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const float sc = e8m0f(bs[d][t]);
#pragma unroll
          for (int j = 0; j < 4; ++j) bop[j][t] = fp4x8_bf16(bw[d][t][j], sc);
        }
        load_b(d, q + KRING);
        const uint16_t *Ab = As[q & 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int mt = 0; mt < MTS; ++mt) {
            const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&Ab[(mt * 16 + l16) * LDA + lq * 32 + j * 8]);
#pragma unroll
            for (int t = 0; t < NTW; ++t)
              acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[j][t], acc[mt][t], 0, 0, 0);
          }
        }
        if (more) store_a((q + 1) & 1);
        __syncthreads();
      }
    }
  }

  // epilogue: acc[mt][t][r] is row mt*16 + 4*lq + r of the pass, feature f[t]
  const uint16_t *bias = g.bias + (int64_t)T.e * g.bias_stride;
  if (PHASE == 0) {
    if (T.tile_on[0]) {
      const float bg = bf16f(bias[T.f[0]]), bu = bf16f(bias[g.I + T.f[0]]);
#pragma unroll
      for (int mt = 0; mt < MTS; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mt * 16 + lq * 4 + r;
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
      for (int mt = 0; mt < MTS; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mt * 16 + lq * 4 + r;
          if (m < T.mrows) {
            const int p = g.perm[T.off + T.m0 + m];
            g.obuf[(int64_t)p * g.H + T.f[t]] = acc[mt][t][r] + bd;
          }
        }
      }
    }
  }
}

template <int PHASE>
__global__ __launch_bounds__(kThreads, 2) void moe_gemm_kernel(GemmArgs g) {
  constexpr int NFB = PHASE == 0 ? 64 : 128;  // features per block
  __shared__ __align__(16) uint16_t As[2][BM * LDA];
  __shared__ int64_t rowoff[BM];
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
  T.l16 = lane & 15;
  T.lq = lane >> 4;
  const int fbase = nt * NFB + wave * (PHASE == 0 ? 16 : 32);
  if (PHASE == 0) {
    T.f[0] = T.f[1] = fbase + T.l16;
    T.nrow[0] = min(T.f[0], g.I - 1);
    T.nrow[1] = g.I + T.nrow[0];
    T.tile_on[0] = T.tile_on[1] = fbase < nfeat;
  } else {
    T.f[0] = fbase + T.l16;
    T.f[1] = T.f[0] + 16;
    T.nrow[0] = min(T.f[0], T.N - 1);
    T.nrow[1] = min(T.f[1], T.N - 1);
    T.tile_on[0] = fbase < nfeat;
    T.tile_on[1] = fbase + 16 < nfeat;
  }
  const int lda_src = PHASE == 0 ? g.H : g.I;

  for (T.m0 = 0; T.m0 < m_e; T.m0 += BM) {
    T.mrows = min(BM, m_e - T.m0);
    __syncthreads();  // the previous pass is done with rowoff and As
    for (int r = threadIdx.x; r < BM; r += kThreads) {
      int64_t o = -1;
      if (r < T.mrows) {
        const int64_t src_row =
            PHASE == 0 ? (int64_t)(g.perm[T.off + T.m0 + r] / g.k) : (int64_t)(T.off + T.m0 + r);
        o = src_row * lda_src;
      }
      rowoff[r] = o;
    }
    __syncthreads();
    switch ((T.mrows + 15) >> 4) {
      case 1: gemm_pass<PHASE, 1>(g, T, As, rowoff); break;
      case 2: gemm_pass<PHASE, 2>(g, T, As, rowoff); break;
      case 3: gemm_pass<PHASE, 3>(g, T, As, rowoff); break;
      case 4: gemm_pass<PHASE, 4>(g, T, As, rowoff); break;
      case 5: gemm_pass<PHASE, 5>(g, T, As, rowoff); break;
      default: gemm_pass<PHASE, 6>(g, T, As, rowoff); break;
    }
  }
}

// ------------------------------------------------------------------ MFMA ceiling
// Eight independent accumulator chains of v_mfma_f32_16x16x32_bf16 per wave, the
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
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{(float)c, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
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
  int64_t offsets, perm, hbuf, obuf, total;
};

WsLayout ws_layout(int H, int I, int n, int k, int E) {
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  WsLayout L;
  const int64_t nk = (int64_t)n * k;
  L.offsets = 0;
  L.perm = up(4ll * (E + 1));
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

int64_t mfma_probe_flops(int blocks, int iters) { return (int64_t)blocks * (kThreads / 64) * iters * 8 * 16 * 16 * 32 * 2; }

bool prefill_supported(int H, int I, int E) { return H % 64 == 0 && I % 64 == 0 && E <= OES_MAX_EXPERTS; }

int64_t prefill_workspace_bytes(int H, int I, int n, int k, int E) { return ws_layout(H, I, n, k, E).total; }

hipError_t launch_prefill_ffn(const PrefillArgs &a, hipStream_t s) {
  if (!prefill_supported(a.H, a.I, a.E)) return hipErrorInvalidValue;
  const WsLayout L = ws_layout(a.H, a.I, a.n, a.k, a.E);
  if (a.ws_bytes < L.total) return hipErrorInvalidValue;
  const int nk = a.n * a.k;
  int32_t *offsets = reinterpret_cast<int32_t *>(a.ws + L.offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(a.ws + L.perm);
  uint16_t *hbuf = reinterpret_cast<uint16_t *>(a.ws + L.hbuf);
  float *obuf = reinterpret_cast<float *>(a.ws + L.obuf);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, s, a.ids, nk, a.E, offsets, perm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemmArgs g;
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
  g.ntiles = (a.I + 63) / 64;
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
  g.ntiles = (a.H + 127) / 128;
  hipLaunchKernelGGL(moe_gemm_kernel<1>, dim3(a.E * g.ntiles), dim3(kThreads), 0, s, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid((a.H / 4 + kThreads - 1) / kThreads, a.n);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(kThreads), 0, s, obuf, a.ids, a.w, a.n, a.k, a.H, a.E, a.y);
  return hipGetLastError();
}

}  // namespace oes
