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
//   block = (expert, 64 output features) x all rows of the expert in passes of
//   128; wave w owns 16 features (gate_up: those 16 gate rows and the matching
//   16 up rows, so silu(g) * u is formed in registers).  K runs in steps of 64
//   (two 32-element MXFP4 blocks).  The A tile (128 rows x 64 k, bf16) is
//   double-buffered in LDS; the B operand needs no LDS: for a 32-element block
//   kb and row n the K-block-major layout [K/32][N][16 B] puts the 8 codes lane l
//   needs in dword l/16 of the 16 bytes at (kb, n), so one dword load per lane
//   (a contiguous 256 B per wave) feeds one MFMA after four fp4 -> bf16 scaled
//   conversions (exact: e2m1 * 2^k is a bf16 number).
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
constexpr int BM = 128;            // rows per pass
constexpr int MT = BM / 16;        // m-tiles per pass
constexpr int BKS = 64;            // k per step: two MXFP4 blocks
constexpr int NF = 64;             // output features per block: 4 waves x 16
constexpr int LDA = BKS + 8;       // padded LDS row, bf16 elements (144 B: spreads banks)
constexpr int kXcds = 8;

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
template <int PHASE>
__global__ __launch_bounds__(kThreads) void moe_gemm_kernel(GemmArgs g) {
  constexpr int NTW = PHASE == 0 ? 2 : 1;  // n-tiles per wave: (gate, up) or one down tile
  __shared__ __align__(16) uint16_t As[2][BM * LDA];
  int e, nt;
  if (g.xcd) {
    const int x = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
    e = x + kXcds * (local / g.ntiles);
    nt = local % g.ntiles;
  } else {
    e = blockIdx.x / g.ntiles;
    nt = blockIdx.x % g.ntiles;
  }
  if (e >= g.E) return;
  const int off = g.offsets[e];
  const int m_e = g.offsets[e + 1] - off;
  if (m_e <= 0) return;
  const int K = PHASE == 0 ? g.H : g.I;    // reduction length
  const int N = PHASE == 0 ? 2 * g.I : g.H;  // weight rows of the matrix
  const int ksteps = K / BKS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int f0 = nt * NF + wave * 16;      // first feature of this wave
  int nrow[NTW];
  nrow[0] = f0 + l16;
  if (NTW == 2) nrow[NTW - 1] = g.I + f0 + l16;  // up row of the same feature
  const uint8_t *blk = g.blocks + (int64_t)e * g.blocks_stride;
  const uint8_t *scl = g.scales + (int64_t)e * g.scales_stride;
  const uint16_t *bias = g.bias + (int64_t)e * g.bias_stride;

  // A-tile loader: thread t moves row t/2, k half (t%2)*32 of the step: 4 x 16 B
  const int arow = threadIdx.x >> 1, akh = (threadIdx.x & 1) * 32;

  for (int m0 = 0; m0 < m_e; m0 += BM) {
    const int mrows = min(BM, m_e - m0);
    const int mtiles = (mrows + 15) >> 4;
    const uint16_t *asrc = nullptr;
    if (arow < mrows) {
      if (PHASE == 0)
        asrc = g.x + (int64_t)(g.perm[off + m0 + arow] / g.k) * g.H + akh;
      else
        asrc = g.hbuf + (int64_t)(off + m0 + arow) * g.I + akh;
    }
    f32x4 acc[MT][NTW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 areg[4];
    uint32_t bw[NTW][2], bs[NTW][2];
    auto load_a = [&](int s) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        areg[q] = asrc ? *reinterpret_cast<const u32x4 *>(asrc + s * BKS + q * 8) : u32x4{0u, 0u, 0u, 0u};
    };
    auto store_a = [&](int buf) {
      u32x4 *d = reinterpret_cast<u32x4 *>(&As[buf][arow * LDA + akh]);
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = areg[q];
    };
    auto load_b = [&](int s) {
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kb = 2 * s + h;
          bw[j][h] = *reinterpret_cast<const uint32_t *>(blk + ((int64_t)kb * N + nrow[j]) * 16 + 4 * lq);
          bs[j][h] = scl[(int64_t)kb * N + nrow[j]];
        }
    };

    load_a(0);
    load_b(0);
    store_a(0);
    __syncthreads();
    for (int s = 0; s < ksteps; ++s) {
      const int cur = s & 1;
      uint32_t cw[NTW][2], cs[NTW][2];
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          cw[j][h] = bw[j][h];
          cs[j][h] = bs[j][h];
        }
      if (s + 1 < ksteps) {
        load_a(s + 1);
        load_b(s + 1);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 bop[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bop[j] = fp4x8_bf16(cw[j][h], e8m0f(cs[j][h]));
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if (i < mtiles) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8 *>(&As[cur][(i * 16 + l16) * LDA + h * 32 + lq * 8]);
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[j], acc[i][j], 0, 0, 0);
          }
        }
      }
      if (s + 1 < ksteps) store_a(cur ^ 1);
      __syncthreads();
    }

    // epilogue: rows 4*lq + r of each m-tile, feature f0 + l16
    const int f = f0 + l16;
    if (PHASE == 0) {
      const float bg = bf16f(bias[f]), bu = bf16f(bias[g.I + f]);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i < mtiles) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + lq * 4 + r;
            if (m < mrows) {
              const float gv = acc[i][0][r] + bg, uv = acc[i][NTW - 1][r] + bu;
              const float hv = gv / (1.f + __expf(-gv)) * uv;
              g.hbuf[(int64_t)(off + m0 + m) * g.I + f] = to_bf16(hv);
            }
          }
        }
      }
    } else {
      const float bd = bf16f(bias[f]);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i < mtiles) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + lq * 4 + r;
            if (m < mrows) {
              const int p = g.perm[off + m0 + m];
              g.obuf[(int64_t)p * g.H + f] = acc[i][0][r] + bd;
            }
          }
        }
      }
    }
    __syncthreads();  // the next pass reuses the LDS tiles
  }
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
  g.ntiles = a.I / NF;
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
  g.ntiles = a.H / NF;
  hipLaunchKernelGGL(moe_gemm_kernel<1>, dim3(a.E * g.ntiles), dim3(kThreads), 0, s, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid((a.H / 4 + kThreads - 1) / kThreads, a.n);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(kThreads), 0, s, obuf, a.ids, a.w, a.n, a.k, a.H, a.E, a.y);
  return hipGetLastError();
}

}  // namespace oes
