// Top-k routing: router logits x . Wg, softmax, top-k, renormalised weights.
//
// The pages name the top-k of each MoE layer (FreeToken MoE benchmark guide §4.3
// routes bs * topk experts per step) but not the router; this is the plain one.
//
// Two launches:
//   route_partial  - split-K GEMV: workgroup s sums rows [s*R, (s+1)*R) of
//                    Wg [H, E] (bf16, row-major) against every token, fp32,
//                    writing partial[s][t][e]; each thread owns one column pair
//                    (a 4-byte load per row, coalesced along E).
//   route_finish   - one wave per token: sums the (at most 32) partials in split
//                    order (deterministic), writes the logits, picks the top-k
//                    by repeated wave argmax (larger logit first, lower index on
//                    ties) and the softmax over the chosen logits.
// route_logits runs route_finish alone on given logits (one split).

#include <math.h>

#include <algorithm>

#include "oes_internal.h"

namespace oes {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kTokBatch = 8;

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ inline float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__global__ __launch_bounds__(kRouteThreads) void route_partial_kernel(const uint16_t *x, const uint32_t *wg2, int n,
                                                                      int H, int E, int rows_per_split,
                                                                      float *partial) {
  __shared__ float red[kRouteThreads * 2 * kTokBatch];
  const int cpt = E >> 1;                      // column pairs
  const int rpp = kRouteThreads / cpt;         // rows processed in parallel
  const int sub = threadIdx.x / cpt, cp = threadIdx.x % cpt;
  const bool active = sub < rpp;
  const int r0 = blockIdx.x * rows_per_split;
  const int r1 = min(H, r0 + rows_per_split);
  for (int t0 = 0; t0 < n; t0 += kTokBatch) {
    const int tn = min(kTokBatch, n - t0);
    float acc[kTokBatch][2];
#pragma unroll
    for (int t = 0; t < kTokBatch; ++t) acc[t][0] = acc[t][1] = 0.f;
    if (active) {
      for (int r = r0 + sub; r < r1; r += rpp) {
        const uint32_t wv = wg2[(int64_t)r * cpt + cp];
        const float w0 = bf16_lo(wv), w1 = bf16_hi(wv);
#pragma unroll
        for (int t = 0; t < kTokBatch; ++t) {
          if (t < tn) {
            const float xv = bf16f(x[(int64_t)(t0 + t) * H + r]);
            acc[t][0] = fmaf(xv, w0, acc[t][0]);
            acc[t][1] = fmaf(xv, w1, acc[t][1]);
          }
        }
      }
    }
    // reduce the rpp row groups through LDS, in fixed order
    __syncthreads();
    if (active) {
#pragma unroll
      for (int t = 0; t < kTokBatch; ++t) {
        red[(sub * kTokBatch + t) * E + 2 * cp] = acc[t][0];
        red[(sub * kTokBatch + t) * E + 2 * cp + 1] = acc[t][1];
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < tn * E; idx += kRouteThreads) {
      const int t = idx / E, e = idx % E;
      float s = 0.f;
      for (int g = 0; g < rpp; ++g) s += red[(g * kTokBatch + t) * E + e];
      partial[((int64_t)blockIdx.x * n + t0 + t) * E + e] = s;
    }
  }
}

struct Cand {
  float v;
  int i;
};

__device__ inline bool better(const Cand &a, const Cand &b) {  // a ranks before b
  return a.v > b.v || (a.v == b.v && a.i < b.i);
}

constexpr int kMaxPerLane = 8;  // E <= 512 experts over 64 lanes

// One wave per token: lane l owns experts l, l + 64, ...; the split partials are
// summed in split order (deterministic), then k rounds of a wave-wide argmax
// (larger logit first, lower index on ties) pick the top-k; lane j keeps the
// j-th pick and writes its id and renormalised weight.
__global__ __launch_bounds__(kRouteThreads) void route_finish_kernel(const float *partial, int splits, int n, int E,
                                                                     int k, float *logits, int32_t *ids, float *w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRouteThreads / 64) + (threadIdx.x >> 6);
  if (t >= n) return;
  const int64_t stride = (int64_t)n * E;
  float z[kMaxPerLane];
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int e = lane + 64 * q;
    float s = 0.f;
    if (e < E) {
      const float *p = partial + (int64_t)t * E + e;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      int sp = 0;
      for (; sp + 4 <= splits; sp += 4) {
        a0 += p[(sp + 0) * stride];
        a1 += p[(sp + 1) * stride];
        a2 += p[(sp + 2) * stride];
        a3 += p[(sp + 3) * stride];
      }
      for (; sp < splits; ++sp) a0 += p[sp * stride];
      s = (a0 + a1) + (a2 + a3);
      if (logits) logits[(int64_t)t * E + e] = s;
    }
    z[q] = s;
  }
  uint32_t taken = 0;
  float myv = 0.f;
  int myi = 0;
  for (int j = 0; j < k; ++j) {
    Cand c{-INFINITY, 0x7fffffff};
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !((taken >> q) & 1u)) {
        Cand o{z[q], e};
        if (c.i == 0x7fffffff || better(o, c)) c = o;
      }
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
      Cand o;
      o.v = __shfl_xor(c.v, d, 64);
      o.i = __shfl_xor(c.i, d, 64);
      if (o.i != 0x7fffffff && (c.i == 0x7fffffff || better(o, c))) c = o;
    }
    if ((c.i & 63) == lane) taken |= 1u << (c.i >> 6);
    if (lane == j) {
      myv = c.v;
      myi = c.i;
    }
  }
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

}  // namespace

int route_splits(int H, int E) {
  const int rpp = kRouteThreads / (E / 2);
  // at most 32 splits (the finishing wave sums them), each a multiple of rpp rows
  int rows = std::max(rpp, (H + 31) / 32);
  rows = (rows + rpp - 1) / rpp * rpp;
  return (H + rows - 1) / rows;
}

static int route_rows_per_split(int H, int E) {
  const int rpp = kRouteThreads / (E / 2);
  int rows = std::max(rpp, (H + 31) / 32);
  return (rows + rpp - 1) / rpp * rpp;
}

hipError_t launch_route(const uint16_t *x, const uint16_t *wg, int n, int H, int E, int k, int32_t *ids, float *w,
                        float *logits, float *partial, hipStream_t s) {
  const int splits = route_splits(H, E);
  const int rows = route_rows_per_split(H, E);
  hipLaunchKernelGGL(route_partial_kernel, dim3(splits), dim3(kRouteThreads), 0, s, x,
                     reinterpret_cast<const uint32_t *>(wg), n, H, E, rows, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_finish_kernel, dim3((n + 3) / 4), dim3(kRouteThreads), 0, s, partial, splits, n, E, k, logits,
                     ids, w);
  return hipGetLastError();
}

hipError_t launch_route_logits(const float *logits, int n, int E, int k, int32_t *ids, float *w, hipStream_t s) {
  hipLaunchKernelGGL(route_finish_kernel, dim3((n + 3) / 4), dim3(kRouteThreads), 0, s, logits, 1, n, E, k,
                     static_cast<float *>(nullptr), ids, w);
  return hipGetLastError();
}

}  // namespace oes
