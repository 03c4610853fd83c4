// Top-k routing: router logits x . Wg, softmax, top-k, renormalised weights.
//
// The pages name the top-k of each MoE layer (FreeToken MoE benchmark guide §4.3
// routes bs * topk experts per step) but not the router; this is the plain one.
//
// Two launches, each one memory round trip deep:
//   route_partial  - split-K GEMV: workgroup s sums rows [s*R, (s+1)*R) of
//                    Wg [H, E] (bf16, row-major) against every token, fp32,
//                    writing partial[s][t][e]; each thread owns one column octet
//                    (a 16-byte load per row, coalesced along E) and up to 16
//                    rows whose loads are all issued before the first multiply.
//   route_finish   - one workgroup per token: all threads sum the partials
//                    (deterministic order), then one wave writes the logits,
//                    picks the top-k by repeated wave argmax (larger logit
//                    first, lower index on ties) and the softmax over the
//                    chosen logits.
// route_logits runs route_finish alone on given logits (one split).

#include <math.h>

#include <algorithm>

#include "oes_internal.h"

namespace oes {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRpt = 16;        // rows per thread, all loads issued at once
constexpr int kMaxTok = 32;     // tokens per pass of the partial kernel

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

struct Cand {
  float v;
  int i;
};

__device__ inline bool better(const Cand &a, const Cand &b) {  // a ranks before b
  return a.v > b.v || (a.v == b.v && a.i < b.i);
}

constexpr int kMaxPerLane = 8;  // E <= 512 experts over 64 lanes

// One workgroup per token.  All 256 threads sum the split partials (thread i
// takes expert i % E and splits i / E, i / E + 256 / E, ... with independent
// loads; the per-thread sums are added in a fixed order through LDS, so the
// result is deterministic).  Then wave 0 picks the top-k by k rounds of a wave
// argmax (larger logit first, lower index on ties); lane j keeps the j-th pick
// and writes its id and renormalised weight.
__global__ __launch_bounds__(kRouteThreads) void route_finish_kernel(const float *partial, int splits, int n, int E,
                                                                     int k, float *logits, int32_t *ids, float *w) {
  __shared__ float zsum[kRouteThreads];
  __shared__ float z[512];
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
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  float zl[kMaxPerLane];
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int e = lane + 64 * q;
    zl[q] = e < E ? z[e] : 0.f;
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
        Cand o{zl[q], e};
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

int route_splits(int H, int E) { return route_geom(H, E).splits; }

hipError_t launch_route(const uint16_t *x, const uint16_t *wg, int n, int H, int E, int k, int32_t *ids, float *w,
                        float *logits, float *partial, hipStream_t s) {
  const RouteGeom geo = route_geom(H, E);
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
