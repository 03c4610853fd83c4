// Decode expert FFN on the slot cache: grouped GEMVs with dequantisation in registers.
//
// FreeToken architecture walk-through §5 (hits are computed straight from the slot
// cache) and §6 (the FP8 block linear and NVFP4 fused MoE kernels this replaces).
// For every token t and routed pair j (slot s = slot_ids[t, j], weight w[t, j]):
//   h_tj = silu(Wg[s] . x_t) * (Wu[s] . x_t)          (gate_up_act kernel)
//   y_t  = sum_j w[t, j] * (Wd[s] . h_tj)               (down_combine kernel)
//
// Both kernels are HBM-bound GEMVs.  A weight row is read as 16-byte chunks;
// a subgroup of G lanes (G | 64) owns one row at a time, lane l taking chunks
// l, l + G, l + 2G, ... so each 16-byte load instruction of a wave covers 64
// consecutive chunks of one or more rows (fully coalesced).  All chunk loads
// of a row (and of its partner row) are issued before any arithmetic.
// Weights are turned into bf16 pairs in registers - exactly, since e4m3 and
// e2m1 values are bf16 numbers - and multiplied with bf16 operands held in LDS
// by v_dot2_f32_bf16 (fp32 accumulation).  Per-block scales (fp8: one fp32 per
// 128x128 block; nvfp4: one e4m3 per 16 elements; q4_0: one fp16 per 32)
// multiply the partial sums; the nvfp4 per-row fp16 global multiplies the
// finished row sum.  A GGUF Q4_0 code q becomes the exact bf16 value 128 + q by
// byte permutation (0x43 is the high byte of bf16 128, whose unit step is 1);
// the dot product of a block then starts from -136 * (sum of its 32 operand
// values), which makes every element count as q - 8.  Lane sums are
// reduced with cross-lane shuffles.  h is kept as bf16 between the kernels.
// y is bf16, rounded to nearest even.

#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "oes_internal.h"

namespace oes {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kMaxQ = 8;   // chunks per lane per pass

// ------------------------------------------------------------------ element decoders
__device__ inline float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), acc,
                                         false);
}
// two e4m3 bytes (bytes 0,1 or 2,3 of w) -> packed bf16 pair (exact)
template <bool HI>
__device__ inline uint32_t fp8_pair_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <bool HI>
__device__ inline f32x2 fp8_pair_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
// the two e2m1 codes of byte B of w (low nibble first) -> packed bf16 pair (exact)
template <int B>
__device__ inline uint32_t fp4_pair_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}
__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline float fp16_to_f32(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }

// bytes 2P and 2P + 1 of n (each a 4-bit code q) -> packed bf16 pair (128 + q_lo, 128 + q_hi)
template <int P>
__device__ inline uint32_t q4_pair_bf16(uint32_t n) {
  // v_perm: selector bytes 0..3 pick bytes of the second operand, 4..7 of the first
  return __builtin_amdgcn_perm(0x43434343u, n, P ? 0x04030402u : 0x04010400u);
}
// sum of the 8 bf16 values in x (fp32)
__device__ inline float sum8_bf16(const u32x4 x, float acc) {
  constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)
  acc = dot2(x.x, kOnes, acc);
  acc = dot2(x.y, kOnes, acc);
  acc = dot2(x.z, kOnes, acc);
  return dot2(x.w, kOnes, acc);
}

// ------------------------------------------------------------------ matrix views
// One matrix (gate_up or down) of the slot banks, for every slot.
struct Mat {
  const uint8_t *codes;   // slot s, row r at codes + s*codes_slot + r*row_bytes
  int64_t codes_slot, row_bytes;
  const uint8_t *scale;   // fp8: f32 [rows/128][K/128]; nvfp4: e4m3 [rows][K/16]; q4_0: fp16 [rows][K/32]
  int64_t scale_slot;
  int32_t scale_ld;
  const uint8_t *glob;    // nvfp4: fp16 [rows]
  int64_t glob_slot;
  int32_t rows, K, C;     // C = chunks per row
};

// Registers of one row's chunks (this lane's share), and the row's nvfp4 global.
struct RowRegs {
  u32x4 w[kMaxQ];
  uint32_t sc[kMaxQ];
  float gl;
};

template <int FMT>
__device__ inline float row_global(const Mat &m, int slot, int row);

template <int FMT, int G>
__device__ inline void load_row(RowRegs &R, const Mat &m, int slot, int row, int lg, int q0, int nq) {
  const u32x4 *p = reinterpret_cast<const u32x4 *>(m.codes + (int64_t)slot * m.codes_slot + (int64_t)row * m.row_bytes);
  R.gl = row_global<FMT>(m, slot, row);  // issued with the weights, used after the lane reduction
#pragma unroll
  for (int q = 0; q < kMaxQ; ++q) {
    if (q < nq) {
      const int c = (q0 + q) * G + lg;
      R.w[q] = __builtin_nontemporal_load(p + c);
      if (FMT == OES_FP8_BLOCK128) {
        const float *s = reinterpret_cast<const float *>(m.scale + (int64_t)slot * m.scale_slot);
        R.sc[q] = __float_as_uint(s[(row >> 7) * m.scale_ld + (c >> 3)]);
      } else if (FMT == OES_NVFP4 || FMT == OES_Q4_0) {  // 16 bits per chunk
        const uint16_t *s = reinterpret_cast<const uint16_t *>(m.scale + (int64_t)slot * m.scale_slot +
                                                               (int64_t)row * m.scale_ld);
        R.sc[q] = s[c];
      }
    }
  }
}

// Dot product of one 16-byte weight chunk (EPC elements) with its bf16 operand
// (EPC/8 16-byte vectors at xo, in LDS or registers); fp8 / nvfp4 / q4_0 block
// scales (packed in sc) are applied here.  xsum (q4_0 only) is the sum of the
// chunk's 32 operand values.
template <int FMT>
__device__ inline float dot_chunk(const u32x4 w, uint32_t sc, const u32x4 *xo, float xsum = 0.f) {
  if (FMT == OES_BF16) {
    const u32x4 x = xo[0];
    float acc = 0.f;
    acc = dot2(w.x, x.x, acc);
    acc = dot2(w.y, x.y, acc);
    acc = dot2(w.z, x.z, acc);
    acc = dot2(w.w, x.w, acc);
    return acc;
  } else if (FMT == OES_FP8_BLOCK128) {
    const u32x4 x0 = xo[0], x1 = xo[1];
    float s = 0.f;
    s = dot2(fp8_pair_bf16<false>(w.x), x0.x, s);
    s = dot2(fp8_pair_bf16<true>(w.x), x0.y, s);
    s = dot2(fp8_pair_bf16<false>(w.y), x0.z, s);
    s = dot2(fp8_pair_bf16<true>(w.y), x0.w, s);
    s = dot2(fp8_pair_bf16<false>(w.z), x1.x, s);
    s = dot2(fp8_pair_bf16<true>(w.z), x1.y, s);
    s = dot2(fp8_pair_bf16<false>(w.w), x1.z, s);
    s = dot2(fp8_pair_bf16<true>(w.w), x1.w, s);
    return s * __uint_as_float(sc);
  } else if (FMT == OES_Q4_0) {
    // one GGUF block: byte j holds element j (low nibble) and element j + 16 (high)
    const u32x4 x0 = xo[0], x1 = xo[1], x2 = xo[2], x3 = xo[3];
    const uint32_t xl[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t xh[8] = {x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    float s = -136.f * xsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = wv[i] & 0x0f0f0f0fu, hi = (wv[i] >> 4) & 0x0f0f0f0fu;
      s = dot2(q4_pair_bf16<0>(lo), xl[2 * i], s);
      s = dot2(q4_pair_bf16<1>(lo), xl[2 * i + 1], s);
      s = dot2(q4_pair_bf16<0>(hi), xh[2 * i], s);
      s = dot2(q4_pair_bf16<1>(hi), xh[2 * i + 1], s);
    }
    return s * fp16_to_f32((uint16_t)sc);
  } else {  // NVFP4: 32 elements, two 16-element scale blocks
    const u32x4 x0 = xo[0], x1 = xo[1], x2 = xo[2], x3 = xo[3];
    float s0 = 0.f, s1 = 0.f;
    s0 = dot2(fp4_pair_bf16<0>(w.x), x0.x, s0);
    s0 = dot2(fp4_pair_bf16<1>(w.x), x0.y, s0);
    s0 = dot2(fp4_pair_bf16<2>(w.x), x0.z, s0);
    s0 = dot2(fp4_pair_bf16<3>(w.x), x0.w, s0);
    s0 = dot2(fp4_pair_bf16<0>(w.y), x1.x, s0);
    s0 = dot2(fp4_pair_bf16<1>(w.y), x1.y, s0);
    s0 = dot2(fp4_pair_bf16<2>(w.y), x1.z, s0);
    s0 = dot2(fp4_pair_bf16<3>(w.y), x1.w, s0);
    s1 = dot2(fp4_pair_bf16<0>(w.z), x2.x, s1);
    s1 = dot2(fp4_pair_bf16<1>(w.z), x2.y, s1);
    s1 = dot2(fp4_pair_bf16<2>(w.z), x2.z, s1);
    s1 = dot2(fp4_pair_bf16<3>(w.z), x2.w, s1);
    s1 = dot2(fp4_pair_bf16<0>(w.w), x3.x, s1);
    s1 = dot2(fp4_pair_bf16<1>(w.w), x3.y, s1);
    s1 = dot2(fp4_pair_bf16<2>(w.w), x3.z, s1);
    s1 = dot2(fp4_pair_bf16<3>(w.w), x3.w, s1);
    const f32x2 scf = fp8_pair_f32<false>(sc);
    return fmaf(s0, scf.x, s1 * scf.y);
  }
}

template <int FMT>
struct Epc;
template <>
struct Epc<OES_BF16> { static constexpr int v = 8; };
template <>
struct Epc<OES_FP8_BLOCK128> { static constexpr int v = 16; };
template <>
struct Epc<OES_NVFP4> { static constexpr int v = 32; };
template <>
struct Epc<OES_Q4_0> { static constexpr int v = 32; };

// Partial dot product of this lane's chunks of a row with a bf16 operand vector in
// LDS (op; q4_0: opsum holds the operand's per-chunk sums).
template <int FMT, int G>
__device__ inline float dot_row(const RowRegs &R, const uint16_t *op, const float *opsum, int lg, int q0, int nq) {
  constexpr int EPC = Epc<FMT>::v;
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxQ; ++q) {
    if (q < nq) {
      const int c = (q0 + q) * G + lg;
      const float xs = FMT == OES_Q4_0 ? opsum[c] : 0.f;
      acc += dot_chunk<FMT>(R.w[q], R.sc[q], reinterpret_cast<const u32x4 *>(op + c * EPC), xs);
    }
  }
  return acc;
}

// Dot products of two rows' chunks (gate and up) with one bf16 operand vector
// in LDS, chunk by chunk: each operand chunk is read once for both rows.
// The weight registers are marked as redefined here (an empty asm), so that a
// caller looping over tokens converts the codes per token instead of hoisting
// every converted chunk out of its loop (which would hold four to eight times
// the registers).
template <int FMT, int G>
__device__ inline void dot_rows2(RowRegs &A, RowRegs &B, const uint16_t *op, const float *opsum, int lg, int nq,
                                 float &da, float &db) {
  constexpr int EPC = Epc<FMT>::v;
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxQ; ++q) {
    if (q < nq) {
      if (FMT != OES_BF16) asm volatile("" : "+v"(A.w[q]), "+v"(B.w[q]));
      const int c = q * G + lg;
      const float xs = FMT == OES_Q4_0 ? opsum[c] : 0.f;
      const u32x4 *xo = reinterpret_cast<const u32x4 *>(op + c * EPC);
      a += dot_chunk<FMT>(A.w[q], A.sc[q], xo, xs);
      b += dot_chunk<FMT>(B.w[q], B.sc[q], xo, xs);
    }
  }
  da = a;
  db = b;
}

template <int G>
__device__ inline float group_sum(float v) {
#pragma unroll
  for (int d = G / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, G);
  return v;
}

// Sums V per-lane values (V items) over a subgroup of G lanes (V <= G, both powers
// of two) with a butterfly that halves the values at every step: (V - 1) +
// log2(G / V) shuffles instead of V * log2(G).  Afterwards the lanes
// [i * G / V, (i + 1) * G / V) of the subgroup all hold the total of item i.
template <int G, int V>
__device__ inline float group_sum_multi(float (&v)[V], int lg) {
  static_assert(V >= 1 && V <= G && (V & (V - 1)) == 0, "V must be a power of two <= G");
#pragma unroll
  for (int h = V / 2, d = G / 2; h >= 1; h >>= 1, d >>= 1) {
    const bool upper = (lg & d) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = upper ? v[i] : v[i + h];
      const float keep = upper ? v[i + h] : v[i];
      v[i] = keep + __shfl_xor(send, d, G);
    }
  }
  float r = v[0];
#pragma unroll
  for (int d = G / V / 2; d > 0; d >>= 1) r += __shfl_xor(r, d, G);
  return r;
}

template <int FMT>
__device__ inline float row_global(const Mat &m, int slot, int row) {
  if (FMT == OES_NVFP4) {
    const uint16_t *g = reinterpret_cast<const uint16_t *>(m.glob + (int64_t)slot * m.glob_slot);
    return fp16_to_f32(g[row]);
  }
  return 1.f;
}

struct KArgs {
  FfnArgs f;
  Mat gu, dn;
};

// Copies `count` bf16 values (count % 8 == 0) from global to LDS.
__device__ inline void stage_bf16(uint16_t *dst, const uint16_t *src, int count) {
  const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
  u32x4 *d = reinterpret_cast<u32x4 *>(dst);
  for (int i = threadIdx.x; i < count / 8; i += kThreads) d[i] = s[i];
}

// ------------------------------------------------------------------ gate_up + act
// grid: (ceil(I / NSG), n*k); each subgroup owns one (gate row, up row) pair.
template <int FMT, int G>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(KArgs ka) {
  extern __shared__ __align__(16) uint16_t xs[];
  const FfnArgs &a = ka.f;
  if (a.gate && *a.gate == 0) return;
  const int p = blockIdx.y;
  const int slot = a.slot_ids[p];
  if (slot < 0) return;
  if (slot >= a.S) {
    if (threadIdx.x == 0) atomicCAS(a.err, 0, (int)OES_ERR_ARG);
    return;
  }
  const int t = p / a.k;
  stage_bf16(xs, a.x + (int64_t)t * a.H, a.H);
  __syncthreads();
  float *xsums = reinterpret_cast<float *>(xs + a.H);  // q4_0: sum of every 32-element block of x
  if (FMT == OES_Q4_0) {
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(xs);
    for (int b = threadIdx.x; b < a.H / 32; b += kThreads) {
      float acc = 0.f;
#pragma unroll
      for (int o = 0; o < 4; ++o) acc = sum8_bf16(xv[4 * b + o], acc);
      xsums[b] = acc;
    }
    __syncthreads();
  }
  constexpr int NSG = kThreads / G;
  const int sg = threadIdx.x / G, lg = threadIdx.x % G;
  const int r = blockIdx.x * NSG + sg;
  if (r >= a.I) return;
  const Mat &m = ka.gu;
  float g = 0.f, u = 0.f, gg = 1.f, gu = 1.f;
  for (int q0 = 0; q0 * G < m.C; q0 += kMaxQ) {
    const int nq = min(kMaxQ, m.C / G - q0);
    RowRegs Rg, Ru;
    load_row<FMT, G>(Rg, m, slot, r, lg, q0, nq);
    load_row<FMT, G>(Ru, m, slot, a.I + r, lg, q0, nq);
    g += dot_row<FMT, G>(Rg, xs, xsums, lg, q0, nq);
    u += dot_row<FMT, G>(Ru, xs, xsums, lg, q0, nq);
    gg = Rg.gl;
    gu = Ru.gl;
  }
  float gu2[2] = {g * gg, u * gu};
  const float tot = group_sum_multi<G, 2>(gu2, lg);  // lanes [0, G/2): gate, [G/2, G): up
  const float other = __shfl_xor(tot, G / 2, G);
  if (lg == 0) {
    g = tot;
    u = other;
    const float hv = g / (1.f + __expf(-g)) * u;
    a.h[(int64_t)p * a.I + r] = f32_to_bf16_rne(hv);
  }
}

// ------------------------------------------------------------------ down + combine
// grid: (ceil(H / RB), n).  Work items are (pair j, row) in pair-major order;
// subgroup sg takes a contiguous run of items, so it mostly keeps one pair: its
// share of h_j (NQ chunks of EPC bf16) is loaded once into registers, and rows
// are processed IB at a time with every weight load issued before the
// arithmetic.  Per-row results over the pairs are combined in pair order
// (deterministic) and written as bf16.
constexpr int kMaxRed = 512;  // RB * k partial results per block (RB <= 16, k <= 32)


template <int FMT, int G, int NQ>
__global__ __launch_bounds__(kThreads) void down_kernel(KArgs ka, int lrb) {
  constexpr int EPC = Epc<FMT>::v;
  constexpr int OPC = EPC / 8;                           // 16-byte operand vectors per chunk
  constexpr int IB0 = NQ >= 2 ? 4 : 8;                  // rows per batch (a power of two)
  constexpr int IB = IB0 < G ? IB0 : G;
  constexpr int NSG = kThreads / G;
  const FfnArgs &a = ka.f;
  if (a.gate && *a.gate == 0) return;
  __shared__ int sl[32];
  __shared__ float wt[32];
  __shared__ float red[kMaxRed];
  const int RB = 1 << lrb;                               // rows per block (a power of two)
  const int t = blockIdx.y;
  const int k = a.k;
  if (threadIdx.x < k) {
    int s = a.slot_ids[t * k + threadIdx.x];
    if (s >= a.S) {
      atomicCAS(a.err, 0, (int)OES_ERR_ARG);
      s = -1;
    }
    sl[threadIdx.x] = s;
    wt[threadIdx.x] = a.w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int sg = threadIdx.x / G, lg = threadIdx.x % G;
  const int r0 = blockIdx.x << lrb;
  const int items = k << lrb;                            // (pair j, row) items, pair-major
  const int ips = (items + NSG - 1) / NSG;
  const int i_end = min(items, (sg + 1) * ips);
  const Mat &m = ka.dn;
  const uint16_t *hbase = a.h + (int64_t)t * k * a.I;
  const uint32_t row_bytes = (uint32_t)m.row_bytes;
  const uint32_t scale_ld = (uint32_t)m.scale_ld;
  u32x4 hreg[NQ][OPC];
  float hsum[NQ];                                        // q4_0: sum of each held chunk of h_j
  int cur_j = -1;
  for (int i0 = sg * ips; i0 < i_end;) {
    const int j = i0 >> lrb;
    const int row0 = r0 + (i0 & (RB - 1));               // rows of a batch are consecutive
    const int cnt = min(IB, min(i_end, (j + 1) << lrb) - i0);
    const int slot = sl[j];
    float acc[IB];
#pragma unroll
    for (int b = 0; b < IB; ++b) acc[b] = 0.f;
    if (slot >= 0) {
      if (j != cur_j) {
        const u32x4 *hp = reinterpret_cast<const u32x4 *>(hbase + (int64_t)j * a.I);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int o = 0; o < OPC; ++o) hreg[q][o] = hp[(q * G + lg) * OPC + o];
        if (FMT == OES_Q4_0) {
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            float acc = 0.f;
#pragma unroll
            for (int o = 0; o < OPC; ++o) acc = sum8_bf16(hreg[q][o], acc);
            hsum[q] = acc;
          }
        }
        cur_j = j;
      }
      // per-batch bases; per-row offsets stay 32-bit
      const uint8_t *cb = m.codes + (int64_t)slot * m.codes_slot;
      const uint8_t *sb = FMT == OES_BF16 ? nullptr : m.scale + (int64_t)slot * m.scale_slot;
      const uint16_t *gb = FMT == OES_NVFP4 ? reinterpret_cast<const uint16_t *>(m.glob + (int64_t)slot * m.glob_slot)
                                            : nullptr;
      u32x4 w[IB][NQ];
      uint32_t sc[IB][NQ];
      float gl[IB];
#pragma unroll
      for (int b = 0; b < IB; ++b) {
        const int row = row0 + b;
        gl[b] = 1.f;
        if (b < cnt && row < a.H) {
          const u32x4 *p = reinterpret_cast<const u32x4 *>(cb + (uint32_t)row * row_bytes);
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int c = q * G + lg;
            w[b][q] = __builtin_nontemporal_load(p + c);
            if (FMT == OES_FP8_BLOCK128)
              sc[b][q] = reinterpret_cast<const uint32_t *>(sb)[(uint32_t)(row >> 7) * scale_ld + (c >> 3)];
            else if (FMT == OES_NVFP4 || FMT == OES_Q4_0)
              sc[b][q] = reinterpret_cast<const uint16_t *>(sb + (uint32_t)row * scale_ld)[c];
            else
              sc[b][q] = 0;
          }
          if (FMT == OES_NVFP4) gl[b] = fp16_to_f32(gb[row]);
        }
      }
#pragma unroll
      for (int b = 0; b < IB; ++b) {
        if (b < cnt && row0 + b < a.H) {
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            acc[b] += dot_chunk<FMT>(w[b][q], sc[b][q], hreg[q], FMT == OES_Q4_0 ? hsum[q] : 0.f);
          acc[b] *= gl[b];  // the row's global multiplies every lane's partial sum
        }
      }
    }
    const float v = group_sum_multi<G, IB>(acc, lg);   // item lg / (G / IB)
    if (lg % (G / IB) == 0) {
      const int b = lg / (G / IB);
      if (b < cnt) red[i0 + b] = (slot >= 0 && row0 + b < a.H) ? v : 0.f;
    }
    i0 += cnt;
  }
  __syncthreads();
  if (threadIdx.x < RB) {
    const int row = r0 + threadIdx.x;
    if (row < a.H) {
      float s = 0.f;
      for (int jj = 0; jj < k; ++jj)
        if (sl[jj] >= 0) s = fmaf(wt[jj], red[(jj << lrb) + threadIdx.x], s);
      a.y[(int64_t)t * a.H + row] = f32_to_bf16_rne(s);
    }
  }
}

// ------------------------------------------------------------------ grouped path (n >= 2)
// With several tokens, pairs routed to the same slot share that expert's rows:
// the rows are streamed once per step and dotted with every such pair's operand,
// so the weight bytes read are u * bytes_per_expert (u = distinct slots) rather
// than one expert per pair.
//   group_pairs  - one workgroup: the distinct slots in ascending order, the
//                  pairs of each (grp), from slot_ids.
//   gate_up      - persistent blocks over (group, 256 / G rows): the group's
//                  tokens' x rows staged in LDS (up to kMG per pass), each
//                  subgroup's gate and up rows read once and dotted with all
//                  of them; h per pair as before.
//   down         - persistent blocks over (group, RB rows): the group's h rows
//                  staged in LDS, each row read once; o per (pair, row) in fp32.
//   combine      - y_t = sum_j w[t, j] * o_tj in pair order, bf16.
// Every pair's dot products have the same reduction order whatever the group
// sizes, so the results do not depend on the order of pairs inside a group.
constexpr int kMG = 8;                   // pairs per LDS pass
constexpr int kGroupThreads = 1024;
constexpr int kSlotsPerThread = OES_MAX_SLOTS / kGroupThreads;

struct GroupView {
  int32_t *count, *slot, *start, *pairs;
};
__device__ inline GroupView group_view(const FfnArgs &a) {
  const int nk = a.n * a.k;
  return {a.grp, a.grp + 4, a.grp + 4 + nk, a.grp + 4 + 2 * nk + 1};
}

__global__ __launch_bounds__(kGroupThreads) void group_pairs_kernel(FfnArgs a) {
  __shared__ int cnt[OES_MAX_SLOTS];   // pairs per slot, then each slot's scatter cursor
  __shared__ int wsum[2][kGroupThreads / 64];
  const GroupView gv = group_view(a);
  const int nk = a.n * a.k, S = a.S;
  if (a.gate && *a.gate == 0) {
    if (threadIdx.x == 0) *gv.count = 0;
    return;
  }
  for (int s = threadIdx.x; s < OES_MAX_SLOTS; s += kGroupThreads) cnt[s] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < nk; p += kGroupThreads) {
    const int s = a.slot_ids[p];
    if (s >= S)
      atomicCAS(a.err, 0, (int)OES_ERR_ARG);
    else if (s >= 0)
      atomicAdd(&cnt[s], 1);
  }
  __syncthreads();
  // thread i owns slots [4i, 4i + 4): exclusive scans, in slot order, of the
  // group flags (count > 0) and of the counts
  int c[kSlotsPerThread], f = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    c[j] = cnt[kSlotsPerThread * threadIdx.x + j];
    f += c[j] > 0;
    tot += c[j];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int fi = f, ti = tot;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int fu = __shfl_up(fi, d), tu = __shfl_up(ti, d);
    if (lane >= d) {
      fi += fu;
      ti += tu;
    }
  }
  if (lane == 63) {
    wsum[0][wave] = fi;
    wsum[1][wave] = ti;
  }
  __syncthreads();
  int fo = fi - f, to = ti - tot;
  for (int w = 0; w < wave; ++w) {
    fo += wsum[0][w];
    to += wsum[1][w];
  }
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    if (c[j] > 0) {
      const int s = kSlotsPerThread * threadIdx.x + j;
      gv.slot[fo] = s;
      gv.start[fo] = to;
      cnt[s] = to;
      ++fo;
      to += c[j];
    }
  }
  if (threadIdx.x == kGroupThreads - 1) {  // its running sums end at the totals
    *gv.count = fo;
    gv.start[fo] = to;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < nk; p += kGroupThreads) {
    const int s = a.slot_ids[p];
    if (s >= 0 && s < S) gv.pairs[atomicAdd(&cnt[s], 1)] = p;
  }
}

// Stages `mg` rows of `len` bf16 values into LDS (row i from src + rowidx(i) * len)
// and, for q4_0, each row's per-32-element sums after them.
template <int FMT, typename RowOf>
__device__ inline void stage_rows(uint16_t *dst, float *sums, const uint16_t *src, int len, int mg, RowOf rowof) {
  const int v = len / 8;
  for (int i = 0; i < mg; ++i) {
    const u32x4 *s = reinterpret_cast<const u32x4 *>(src + (int64_t)rowof(i) * len);
    u32x4 *d = reinterpret_cast<u32x4 *>(dst + i * len);
    for (int j = threadIdx.x; j < v; j += kThreads) d[j] = s[j];
  }
  if (FMT == OES_Q4_0) {
    __syncthreads();
    const int nb = len / 32;
    for (int b = threadIdx.x; b < mg * nb; b += kThreads) {
      const u32x4 *xv = reinterpret_cast<const u32x4 *>(dst) + 4 * b;  // rows are whole blocks
      float acc = 0.f;
#pragma unroll
      for (int o = 0; o < 4; ++o) acc = sum8_bf16(xv[o], acc);
      sums[b] = acc;
    }
  }
}

template <int FMT, int G>
__global__ __launch_bounds__(kThreads) void gate_up_grouped_kernel(KArgs ka, int mgmax) {
  extern __shared__ __align__(16) uint16_t xs[];  // mgmax x rows of H, then q4_0 block sums
  __shared__ int sp[kMG];
  const FfnArgs &a = ka.f;
  if (a.gate && *a.gate == 0) return;
  const GroupView gv = group_view(a);
  const int ng = *gv.count;
  constexpr int NSG = kThreads / G;
  const int rblk = (a.I + NSG - 1) / NSG;
  const int sg = threadIdx.x / G, lg = threadIdx.x % G;
  float *xsums = reinterpret_cast<float *>(xs + (size_t)mgmax * a.H);
  const int nb = a.H / 32;
  const Mat &m = ka.gu;
  const int nqt = m.C / G;  // chunks per lane of a row
  for (int item = blockIdx.x; item < ng * rblk; item += gridDim.x) {
    const int g = item / rblk;
    const int r = (item - g * rblk) * NSG + sg;
    const int slot = gv.slot[g], p0 = gv.start[g], p1 = gv.start[g + 1];
    for (int pp = p0; pp < p1; pp += mgmax) {
      const int mg = min(mgmax, p1 - pp);
      __syncthreads();  // the previous pass is done with xs and sp
      if ((int)threadIdx.x < mg) sp[threadIdx.x] = gv.pairs[pp + threadIdx.x];
      __syncthreads();
      stage_rows<FMT>(xs, xsums, a.x, a.H, mg, [&](int i) { return sp[i] / a.k; });
      __syncthreads();
      if (r < a.I) {
        // the rows stay in registers (one pass: C / G <= kMaxQ, checked at launch)
        // while every staged token is dotted with them
        RowRegs Rg, Ru;
        load_row<FMT, G>(Rg, m, slot, r, lg, 0, nqt);
        load_row<FMT, G>(Ru, m, slot, a.I + r, lg, 0, nqt);
#pragma unroll 1
        for (int i = 0; i < mg; ++i) {
          float dg, du;
          dot_rows2<FMT, G>(Rg, Ru, xs + i * a.H, xsums + i * nb, lg, nqt, dg, du);
          float gu2[2] = {dg * Rg.gl, du * Ru.gl};
          const float tot = group_sum_multi<G, 2>(gu2, lg);  // lanes [0, G/2): gate, [G/2, G): up
          const float other = __shfl_xor(tot, G / 2, G);
          if (lg == 0) a.h[(int64_t)sp[i] * a.I + r] = f32_to_bf16_rne(tot / (1.f + __expf(-tot)) * other);
        }
      }
    }
  }
}

template <int FMT, int G, int NQ>
__global__ __launch_bounds__(kThreads) void down_grouped_kernel(KArgs ka, int mgmax) {
  extern __shared__ __align__(16) uint16_t hs[];  // mgmax h rows of I, then q4_0 block sums
  __shared__ int sp[kMG];
  constexpr int EPC = Epc<FMT>::v;
  constexpr int IB = 4;                 // consecutive rows per subgroup
  constexpr int NSG = kThreads / G;
  constexpr int RB = NSG * IB;          // rows per work item
  const FfnArgs &a = ka.f;
  if (a.gate && *a.gate == 0) return;
  const GroupView gv = group_view(a);
  const int ng = *gv.count;
  const int rblk = (a.H + RB - 1) / RB;
  const int sg = threadIdx.x / G, lg = threadIdx.x % G;
  float *hsums = reinterpret_cast<float *>(hs + (size_t)mgmax * a.I);
  const int nb = a.I / 32;
  const Mat &m = ka.dn;
  const uint32_t row_bytes = (uint32_t)m.row_bytes, scale_ld = (uint32_t)m.scale_ld;
  for (int item = blockIdx.x; item < ng * rblk; item += gridDim.x) {
    const int g = item / rblk;
    const int row0 = (item - g * rblk) * RB + sg * IB;
    const int slot = gv.slot[g], p0 = gv.start[g], p1 = gv.start[g + 1];
    const uint8_t *cb = m.codes + (int64_t)slot * m.codes_slot;
    const uint8_t *sb = FMT == OES_BF16 ? nullptr : m.scale + (int64_t)slot * m.scale_slot;
    const uint16_t *gb =
        FMT == OES_NVFP4 ? reinterpret_cast<const uint16_t *>(m.glob + (int64_t)slot * m.glob_slot) : nullptr;
    for (int pp = p0; pp < p1; pp += mgmax) {
      const int mg = min(mgmax, p1 - pp);
      __syncthreads();
      if ((int)threadIdx.x < mg) sp[threadIdx.x] = gv.pairs[pp + threadIdx.x];
      __syncthreads();
      // the rows' weights are loaded before the staging waits, so the two overlap
      u32x4 w[IB][NQ];
      uint32_t sc[IB][NQ];
      float gl[IB];
#pragma unroll
      for (int b = 0; b < IB; ++b) {
        const int row = min(row0 + b, a.H - 1);  // rows past H repeat the last row; never stored
        const u32x4 *p = reinterpret_cast<const u32x4 *>(cb + (uint32_t)row * row_bytes);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int c = q * G + lg;
          w[b][q] = __builtin_nontemporal_load(p + c);
          if (FMT == OES_FP8_BLOCK128)
            sc[b][q] = reinterpret_cast<const uint32_t *>(sb)[(uint32_t)(row >> 7) * scale_ld + (c >> 3)];
          else if (FMT == OES_NVFP4 || FMT == OES_Q4_0)
            sc[b][q] = reinterpret_cast<const uint16_t *>(sb + (uint32_t)row * scale_ld)[c];
          else
            sc[b][q] = 0;
        }
        gl[b] = FMT == OES_NVFP4 ? fp16_to_f32(gb[row]) : 1.f;
      }
      stage_rows<FMT>(hs, hsums, a.h, a.I, mg, [&](int i) { return sp[i]; });
      __syncthreads();
#pragma unroll 1
      for (int i = 0; i < mg; ++i) {
        {
          const uint16_t *hv = hs + i * a.I;
          float acc[IB];
#pragma unroll
          for (int b = 0; b < IB; ++b) acc[b] = 0.f;
#pragma unroll
          for (int q = 0; q < NQ; ++q) {  // each h chunk is read once for all the rows
            if (FMT != OES_BF16) {   // converted per token, not hoisted out of the token loop
#pragma unroll
              for (int b = 0; b < IB; ++b) asm volatile("" : "+v"(w[b][q]));
            }
            const int c = q * G + lg;
            const u32x4 *ho = reinterpret_cast<const u32x4 *>(hv + c * EPC);
            const float hsum = FMT == OES_Q4_0 ? hsums[i * nb + c] : 0.f;
#pragma unroll
            for (int b = 0; b < IB; ++b) acc[b] += dot_chunk<FMT>(w[b][q], sc[b][q], ho, hsum);
          }
#pragma unroll
          for (int b = 0; b < IB; ++b) acc[b] *= gl[b];
          const float v = group_sum_multi<G, IB>(acc, lg);  // row lg / (G / IB)
          const int b = lg / (G / IB);
          if (lg % (G / IB) == 0 && row0 + b < a.H) a.o[(int64_t)sp[i] * a.H + row0 + b] = v;
        }
      }
    }
  }
}

// y[t, c..c+3] = sum_j w[t, j] * o[t k + j, c..c+3] over the pairs with a slot, in j order.
__global__ __launch_bounds__(256) void combine_pairs_kernel(FfnArgs a) {
  if (a.gate && *a.gate == 0) return;
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= a.H) return;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int j = 0; j < a.k; ++j) {
    const int p = t * a.k + j;
    const int slot = a.slot_ids[p];
    if (slot < 0 || slot >= a.S) continue;
    const float wt = a.w[p];
    const float4 o = *reinterpret_cast<const float4 *>(a.o + (int64_t)p * a.H + c);
    s0 = fmaf(wt, o.x, s0);
    s1 = fmaf(wt, o.y, s1);
    s2 = fmaf(wt, o.z, s2);
    s3 = fmaf(wt, o.w, s3);
  }
  uint16_t *yr = a.y + (int64_t)t * a.H + c;
  yr[0] = f32_to_bf16_rne(s0);
  yr[1] = f32_to_bf16_rne(s1);
  yr[2] = f32_to_bf16_rne(s2);
  yr[3] = f32_to_bf16_rne(s3);
}

// ------------------------------------------------------------------ dispatch
int pick_group(int C) {
  if (C % 64 == 0) return 64;
  if (C % 32 == 0) return 32;
  if (C % 16 == 0) return 16;
  if (C % 8 == 0) return 8;
  return 0;
}

// down subgroups: at least one subgroup per routed pair (G <= 256 / k), each lane
// holding at most 4 chunks of a row, so a block's rows x pairs split into one
// batch per subgroup.
int pick_group_dn(int C, int k) {
  for (int g = 64; g >= 8; g /= 2)
    if (C % g == 0 && C / g <= 4 && g * k <= kThreads) return g;
  for (int g = 64; g >= 8; g /= 2)
    if (C % g == 0 && C / g <= 4) return g;
  return 0;
}

// gate_up subgroups: the smallest G whose share is at most kMaxQ chunks per lane
// (each lane keeps up to 2 x kMaxQ 16-byte loads, gate and up rows, in flight)
// and whose grid still has 512 blocks (two per CU); short rows (few chunks) take
// a wider G instead, trading loads in flight per lane for blocks.
int pick_group_gu(int C, int I, int pairs) {
  int last = 0;
  for (int g = 8; g <= 64; g *= 2) {
    if (C % g || C / g > kMaxQ) continue;
    last = g;
    const int64_t blocks = (int64_t)((I + kThreads / g - 1) / (kThreads / g)) * pairs;
    if (blocks >= 512) return g;
  }
  return last ? last : pick_group(C);
}

int epc_of(int fmt) {
  return fmt == OES_BF16 ? 8 : fmt == OES_FP8_BLOCK128 ? 16 : (fmt == OES_NVFP4 || fmt == OES_Q4_0) ? 32 : 0;
}

Mat make_mat(const FfnArgs &a, bool down) {
  Mat m = {};
  const int fmt = a.format;
  const int rows = down ? a.H : 2 * a.I;
  const int K = down ? a.I : a.H;
  m.rows = rows;
  m.K = K;
  m.C = K / epc_of(fmt);
  int bc = 0, bs = -1, bg = -1;
  if (fmt == OES_BF16) {
    bc = down ? 1 : 0;
  } else if (fmt == OES_FP8_BLOCK128 || fmt == OES_Q4_0) {
    bc = down ? 2 : 0;
    bs = bc + 1;
  } else {
    bc = down ? 3 : 0;
    bs = bc + 1;
    bg = bc + 2;
  }
  m.codes = a.bank[bc];
  m.codes_slot = a.row_bytes[bc];
  m.row_bytes = m.codes_slot / rows;
  if (bs >= 0) {
    m.scale = a.bank[bs];
    m.scale_slot = a.row_bytes[bs];
    m.scale_ld = fmt == OES_FP8_BLOCK128 ? K / 128 : K / 16;  // nvfp4 / q4_0: bytes per row
  }
  if (bg >= 0) {
    m.glob = a.bank[bg];
    m.glob_slot = a.row_bytes[bg];
  }
  return m;
}

template <int FMT, int G>
hipError_t launch_gate_up_g(const KArgs &ka, hipStream_t s) {
  const FfnArgs &a = ka.f;
  constexpr int NSG = kThreads / G;
  dim3 grid((a.I + NSG - 1) / NSG, a.n * a.k);
  const size_t lds = (size_t)a.H * 2 + (FMT == OES_Q4_0 ? (size_t)(a.H / 32) * 4 : 0);
  hipLaunchKernelGGL((gate_up_kernel<FMT, G>), grid, dim3(kThreads), lds, s, ka);
  return hipGetLastError();
}

// Rows per block, a power of two in [1, 16]: the largest whose grid keeps about
// three blocks per CU (768).  Every block reads each of its pairs' h rows once
// per subgroup that takes that pair, so larger blocks cut that re-read; where
// several subgroups share a pair (narrow G, small k) the re-read weighs more and
// two blocks per CU (512) is the target.  Both targets were picked by timing
// every (G, rows) choice on the decode workloads' shapes at 1, 2 and 8 tokens.
int down_rows_per_block(int G, int k, int H, int n) {
  const int64_t target = kThreads / G > k ? 512 : 768;
  int rb = 16;
  while (rb > 1 && (int64_t)((H + rb - 1) / rb) * n < target) rb >>= 1;
  return rb;
}

template <int FMT, int G, int NQ>
hipError_t launch_down_gq(const KArgs &ka, hipStream_t s) {
  const FfnArgs &a = ka.f;
  const int rb = down_rows_per_block(G, a.k, a.H, a.n);
  int lrb = 0;
  while ((1 << lrb) < rb) ++lrb;
  dim3 grid((a.H + rb - 1) / rb, a.n);
  hipLaunchKernelGGL((down_kernel<FMT, G, NQ>), grid, dim3(kThreads), 0, s, ka, lrb);
  return hipGetLastError();
}

template <int FMT, int G>
hipError_t launch_down_g(const KArgs &ka, hipStream_t s) {
  switch (ka.dn.C / G) {
    case 1: return launch_down_gq<FMT, G, 1>(ka, s);
    case 2: return launch_down_gq<FMT, G, 2>(ka, s);
    case 3: return launch_down_gq<FMT, G, 3>(ka, s);
    case 4: return launch_down_gq<FMT, G, 4>(ka, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ grouped dispatch
// down subgroups of the grouped path: the widest G whose share of a row is at
// most 4 chunks per lane.
int pick_group_dn_grouped(int C) {
  for (int g = 64; g >= 8; g /= 2)
    if (C % g == 0 && C / g <= 4) return g;
  return 0;
}

// Pairs per LDS pass: at most kMG, and at most 32 KiB of staged bf16 rows.
int group_mg(int len) { return std::max(1, std::min(kMG, 32768 / (2 * len))); }

size_t staged_lds(int fmt, int mg, int len) {
  return (size_t)mg * len * 2 + (fmt == OES_Q4_0 ? (size_t)mg * (len / 32) * 4 : 0);
}

// Persistent grid: every CU holds as many blocks as fit, capped by the work items.
template <typename K>
int persistent_blocks(K kernel, size_t lds, int64_t items) {
  int dev = 0, cus = 0, per_cu = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  (void)hipGetLastError();
  return (int)std::max<int64_t>(1, std::min<int64_t>(items, (int64_t)cus * per_cu));
}

template <int FMT, int G>
hipError_t launch_gate_up_grouped(const KArgs &ka, hipStream_t s) {
  const FfnArgs &a = ka.f;
  constexpr int NSG = kThreads / G;
  const int mg = group_mg(a.H);
  const size_t lds = staged_lds(FMT, mg, a.H);
  const int64_t items = (int64_t)a.n * a.k * ((a.I + NSG - 1) / NSG);  // distinct slots <= pairs
  auto kern = gate_up_grouped_kernel<FMT, G>;
  hipLaunchKernelGGL(kern, dim3(persistent_blocks(kern, lds, items)), dim3(kThreads), lds, s, ka, mg);
  return hipGetLastError();
}

template <int FMT, int G, int NQ>
hipError_t launch_down_grouped_gq(const KArgs &ka, hipStream_t s) {
  const FfnArgs &a = ka.f;
  constexpr int RB = (kThreads / G) * 4;
  const int mg = group_mg(a.I);
  const size_t lds = staged_lds(FMT, mg, a.I);
  const int64_t items = (int64_t)a.n * a.k * ((a.H + RB - 1) / RB);
  auto kern = down_grouped_kernel<FMT, G, NQ>;
  hipLaunchKernelGGL(kern, dim3(persistent_blocks(kern, lds, items)), dim3(kThreads), lds, s, ka, mg);
  return hipGetLastError();
}

template <int FMT, int G>
hipError_t launch_down_grouped_g(const KArgs &ka, hipStream_t s) {
  switch (ka.dn.C / G) {
    case 1: return launch_down_grouped_gq<FMT, G, 1>(ka, s);
    case 2: return launch_down_grouped_gq<FMT, G, 2>(ka, s);
    case 3: return launch_down_grouped_gq<FMT, G, 3>(ka, s);
    case 4: return launch_down_grouped_gq<FMT, G, 4>(ka, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT>
hipError_t launch_fmt_grouped(const KArgs &ka, hipStream_t s) {
  const FfnArgs &a = ka.f;
  hipLaunchKernelGGL(group_pairs_kernel, dim3(1), dim3(kGroupThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (pick_group_gu(ka.gu.C, a.I, a.n * a.k)) {
    case 64: e = launch_gate_up_grouped<FMT, 64>(ka, s); break;
    case 32: e = launch_gate_up_grouped<FMT, 32>(ka, s); break;
    case 16: e = launch_gate_up_grouped<FMT, 16>(ka, s); break;
    case 8: e = launch_gate_up_grouped<FMT, 8>(ka, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  switch (pick_group_dn_grouped(ka.dn.C)) {
    case 64: e = launch_down_grouped_g<FMT, 64>(ka, s); break;
    case 32: e = launch_down_grouped_g<FMT, 32>(ka, s); break;
    case 16: e = launch_down_grouped_g<FMT, 16>(ka, s); break;
    case 8: e = launch_down_grouped_g<FMT, 8>(ka, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_pairs_kernel, dim3((a.H / 4 + 255) / 256, a.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

// The grouped path costs two more launches and the o round trip; it pays when
// experts repeat enough.  The repeats expected of uniform top-k routing over E
// experts, n k - E (1 - (1 - k / E)^n), must save at least 128 MB of weight reads
// (measured on the decode workloads: bf16 H=2048 at 32 tokens 346 -> 180 us and
// fp8 H=4096 at 16 tokens 356 -> 324 us grouped; nvfp4 H=7168 at 4 tokens, Q4_0
// H=2048 at 8 and bf16 H=2048 at 8 no faster or slower), and a subgroup must hold
// a whole gate / up row in registers.
bool use_grouped(const KArgs &ka) {
  const FfnArgs &a = ka.f;
  if (a.n < 2 || a.path == OES_FFN_PER_PAIR) return false;
  if (ka.gu.C > 64 * kMaxQ || ka.gu.C / pick_group_gu(ka.gu.C, a.I, a.n * a.k) > kMaxQ) return false;
  if (a.path == OES_FFN_GROUPED) return true;
  if (a.E <= 0) return false;
  const double E = a.E, nk = (double)a.n * a.k;
  const double unique = E * (1.0 - pow(1.0 - std::min(1.0, a.k / E), (double)a.n));
  int64_t bpe = 0;
  for (int b = 0; b < OES_MAX_BANKS; ++b) bpe += a.row_bytes[b];
  return (nk - unique) * (double)bpe >= 128.0 * (1 << 20);
}

template <int FMT>
hipError_t launch_fmt(const KArgs &ka, hipStream_t s) {
  if (use_grouped(ka)) return launch_fmt_grouped<FMT>(ka, s);
  hipError_t e;
  switch (pick_group_gu(ka.gu.C, ka.f.I, ka.f.n * ka.f.k)) {
    case 64: e = launch_gate_up_g<FMT, 64>(ka, s); break;
    case 32: e = launch_gate_up_g<FMT, 32>(ka, s); break;
    case 16: e = launch_gate_up_g<FMT, 16>(ka, s); break;
    case 8: e = launch_gate_up_g<FMT, 8>(ka, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  switch (pick_group_dn(ka.dn.C, ka.f.k)) {
    case 64: return launch_down_g<FMT, 64>(ka, s);
    case 32: return launch_down_g<FMT, 32>(ka, s);
    case 16: return launch_down_g<FMT, 16>(ka, s);
    case 8: return launch_down_g<FMT, 8>(ka, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ decoder check
__global__ void debug_decode_kernel(int elem, const uint8_t *codes, int n, float *out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (elem == OES_ELEM_FP4X2) {
    // i indexes a byte: elements 2i and 2i+1
    if (2 * i >= n) return;
    const uint32_t word = codes[i];
    const uint32_t pr = fp4_pair_bf16<0>(word);
    out[2 * i] = bf16_to_f32(pr & 0xffffu);
    if (2 * i + 1 < n) out[2 * i + 1] = bf16_to_f32(pr >> 16);
    return;
  }
  if (i >= n) return;
  if (elem == OES_ELEM_Q4X2) {
    // element i: block i / 32, position j; code byte j % 16 of the block, low
    // nibble for j < 16; decoded by the FFN's permutation, minus the 128 + 8 offset
    const int j = i % 32, bj = j % 16;
    const uint32_t dw = reinterpret_cast<const uint32_t *>(codes + (i / 32) * 16)[bj / 4];
    const uint32_t nib = j < 16 ? dw & 0x0f0f0f0fu : (dw >> 4) & 0x0f0f0f0fu;
    const uint32_t pr = (bj % 4) < 2 ? q4_pair_bf16<0>(nib) : q4_pair_bf16<1>(nib);
    out[i] = bf16_to_f32(bj % 2 ? pr >> 16 : pr & 0xffffu) - 136.f;
    return;
  }
  if (elem == OES_ELEM_E4M3) {
    out[i] = fp8_pair_f32<false>((uint32_t)codes[i]).x;
  } else if (elem == OES_ELEM_E8M0) {
    const uint32_t e = codes[i];
    out[i] = e == 255 ? __uint_as_float(0x7fc00000u) : (e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23));
  } else if (elem == OES_ELEM_BF16) {
    out[i] = bf16_to_f32(reinterpret_cast<const uint16_t *>(codes)[i]);
  } else if (elem == OES_ELEM_FP16) {
    out[i] = fp16_to_f32(reinterpret_cast<const uint16_t *>(codes)[i]);
  }
}

// ------------------------------------------------------------------ hybrid combine
__global__ __launch_bounds__(256) void add_to_bf16_kernel(uint16_t *y, const float *add, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    y[i] = f32_to_bf16_rne(bf16_to_f32(y[i]) + add[i]);
}

}  // namespace

hipError_t launch_add_to_bf16(uint16_t *y, const float *add, int64_t count, hipStream_t s) {
  const int blocks = (int)std::min<int64_t>(1024, (count + 255) / 256);
  hipLaunchKernelGGL(add_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, y, add, count);
  return hipGetLastError();
}

bool expert_ffn_supported(int format, int H, int I, int k) {
  const int epc = epc_of(format);
  if (!epc) return false;
  if (H % epc || I % epc) return false;
  const int gu = pick_group_gu(H / epc, I, k), dn = pick_group_dn(I / epc, k);
  if (!gu || !dn || !pick_group_dn_grouped(I / epc)) return false;  // down: at most 4 chunks per lane in registers
  if (H % 4) return false;  // combine: four columns per thread
  if (H > 16384) return false;          // x row staged in LDS by gate_up
  if (k > 32 || 16 * k > kMaxRed) return false;
  return true;
}

// Workspace: h bf16 [n k, I]; for n >= 2 also o fp32 [n k, H] and the grouping
// (count, then slot [n k], start [n k + 1], pairs [n k] as int32), each part
// 256-byte aligned.
static int64_t ws_round(int64_t v) { return (v + 255) / 256 * 256; }

int64_t expert_ffn_workspace_bytes(int n, int k, int H, int I) {
  const int64_t nk = (int64_t)n * k;
  int64_t bytes = ws_round(2 * nk * I);
  if (n >= 2) bytes += ws_round(4 * nk * H) + ws_round(4 * (4 + 3 * nk + 1));
  return bytes;
}

void expert_ffn_carve(FfnArgs &a, void *workspace) {
  uint8_t *p = static_cast<uint8_t *>(workspace);
  const int64_t nk = (int64_t)a.n * a.k;
  a.h = reinterpret_cast<uint16_t *>(p);
  p += ws_round(2 * nk * a.I);
  a.o = nullptr;
  a.grp = nullptr;
  if (a.n >= 2) {
    a.o = reinterpret_cast<float *>(p);
    p += ws_round(4 * nk * a.H);
    a.grp = reinterpret_cast<int32_t *>(p);
  }
}

hipError_t launch_expert_ffn(const FfnArgs &a, hipStream_t s) {
  KArgs ka;
  ka.f = a;
  ka.gu = make_mat(a, false);
  ka.dn = make_mat(a, true);
  switch (a.format) {
    case OES_BF16: return launch_fmt<OES_BF16>(ka, s);
    case OES_FP8_BLOCK128: return launch_fmt<OES_FP8_BLOCK128>(ka, s);
    case OES_NVFP4: return launch_fmt<OES_NVFP4>(ka, s);
    case OES_Q4_0: return launch_fmt<OES_Q4_0>(ka, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------ no-alloc scratch
// Workspace of oes_expert_ffn_noalloc: one array per GPU, alive until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host the name
// is only a stand-in); it passes the device address looked up here, once per
// device with that device current.
static __device__ __align__(256) uint8_t scratch[OES_FFN_NOALLOC_SCRATCH_BYTES];

hipError_t ffn_noalloc_scratch(int device, void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t launch_debug_decode(int elem, const uint8_t *codes, int n, float *out, hipStream_t s) {
  const int items = elem == OES_ELEM_FP4X2 ? (n + 1) / 2 : n;
  hipLaunchKernelGGL(debug_decode_kernel, dim3((items + 255) / 256), dim3(256), 0, s, elem, codes, n, out);
  return hipGetLastError();
}

}  // namespace oes
