// CPU MoE executor of the hybrid backend: the experts a hybrid step leaves
// unfetched (slot -1) are computed on the host cores, straight from the pinned
// host banks, while the GPU copies the fetched ones.
//
// FreeToken architecture walk-through §5 (PCIe-bound experts are computed by
// the CPU with AVX-512 GEMVs, the fetch split following the measured
// bandwidths) and FreeToken MoE benchmark guide §5.2 and §5.4 (the CPU MoE
// kernel, its bandwidth against the PCIe gather, the decision rule and the
// -1 experts of ensure_experts_hybrid).
//
// One call, for the CPU pairs (t, j) (slot_ids[t, j] < 0, expert e = ids[t, j]):
//   pass 1: h_tj[r] = silu(Wg_e[r] . x_t) * (Wu_e[r] . x_t), rounded to bf16;
//           the flattened (pair, r) space is cut into one contiguous range per
//           thread;
//   pass 2: y[t][r] = sum_j w[t, j] * (Wd_e[r] . h_tj) over the CPU pairs in
//           (t, j) order; output rows are cut into one range per thread.
// The summation order depends on neither the thread count nor the timing.
// Weights are read from the host banks 32 or 64 elements at a time and turned
// into bf16 exactly (bf16 as is; e2m1 and q - 8 through a 32-entry table with
// vpermw), multiplied with the bf16 operand by vdpbf16ps (fp32 accumulate),
// scaled per block (nvfp4: e4m3 per 16, then the fp16 row global; q4_0: fp16
// per 32).  Needs AVX-512 F/BW/VL/BF16 and F16C; without them the executor is
// not created (OES_ERR_UNSUPPORTED).

#include <immintrin.h>
#include <math.h>
#include <sched.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "oes.h"

namespace oes {
oes_status set_error(oes_status st, const char *msg);  // host_common.cpp: thread-local message
}

namespace {

oes_status fail(oes_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
oes_status fail(oes_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return oes::set_error(st, buf);
}

// ------------------------------------------------------------------ thread pool
// Workers spin briefly on a generation counter, then sleep on a condition
// variable; the calling thread is worker 0.
class Pool {
 public:
  explicit Pool(int n) : n_(n) {
    for (int i = 1; i < n_; ++i) th_.emplace_back([this, i] { loop(i); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> l(m_);
      stop_.store(true, std::memory_order_release);
    }
    cv_.notify_all();
    for (auto &t : th_) t.join();
  }
  int size() const { return n_; }

  // fn(tid, n) on every worker; returns when all have returned.
  void run(const std::function<void(int, int)> &fn) {
    if (n_ == 1) {
      fn(0, 1);
      return;
    }
    fn_ = &fn;
    left_.store(n_ - 1, std::memory_order_relaxed);
    {
      std::lock_guard<std::mutex> l(m_);
      gen_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    fn(0, n_);
    for (int spin = 0; left_.load(std::memory_order_acquire) != 0; ++spin) {
      if (spin < kSpin) {
        _mm_pause();
      } else {
        std::unique_lock<std::mutex> l(m_);
        done_.wait(l, [&] { return left_.load(std::memory_order_acquire) == 0; });
      }
    }
  }

 private:
  // a few tens of microseconds: enough to bridge the two passes of a call, short
  // enough that idle workers stop using the CPU quota soon after a call
  static constexpr int kSpin = 2000;
  void loop(int tid) {
    uint64_t seen = 0;
    for (;;) {
      uint64_t g;
      for (int spin = 0; (g = gen_.load(std::memory_order_acquire)) == seen; ++spin) {
        if (stop_.load(std::memory_order_acquire)) return;
        if (spin < kSpin) {
          _mm_pause();
        } else {
          std::unique_lock<std::mutex> l(m_);
          cv_.wait(l, [&] {
            return gen_.load(std::memory_order_acquire) != seen || stop_.load(std::memory_order_acquire);
          });
        }
      }
      if (stop_.load(std::memory_order_acquire)) return;
      seen = g;
      (*fn_)(tid, n_);
      if (left_.fetch_sub(1, std::memory_order_acq_rel) == 1) {
        std::lock_guard<std::mutex> l(m_);
        done_.notify_one();
      }
    }
  }
  int n_;
  std::vector<std::thread> th_;
  std::mutex m_;
  std::condition_variable cv_, done_;
  const std::function<void(int, int)> *fn_ = nullptr;
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> left_{0};
  std::atomic<bool> stop_{false};
};

// ------------------------------------------------------------------ numbers
float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
// bf16 bits of f, rounded to nearest even (NaN kept quiet)
uint16_t bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// OCP e4m3: bias 7, no infinities, S.1111.111 is NaN
float e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return bits_f32(0x7fc00000u);
  const float mag = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.f + m / 8.f, e - 7);
  return s ? -mag : mag;
}
// OCP e2m1: bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives
float e2m1_value(uint8_t c) {
  const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  const float mag = e == 0 ? 0.5f * m : ldexpf(1.f + 0.5f * m, e - 1);
  return s ? -mag : mag;
}

#define OES_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512bf16,f16c,fma")))

struct Tables {
  alignas(64) uint16_t e2m1[32];  // bf16 of each e2m1 code (entries 16..31 unused)
  alignas(64) uint16_t q4[32];    // bf16 of q - 8 for each 4-bit code
  float e4m3[256];
};

OES_AVX512 inline __m512 dp(__m512 acc, __m512i a, __m512i b) {
  return _mm512_dpbf16_ps(acc, (__m512bh)a, (__m512bh)b);
}

OES_AVX512 inline float fp16_value(uint16_t h) { return _cvtsh_ss(h); }

// bf16 row (K elements, K % 8 == 0) . bf16 vector
OES_AVX512 float dot_bf16(const uint16_t *w, const uint16_t *x, int K) {
  __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
  int k = 0;
  for (; k + 64 <= K; k += 64) {
    a0 = dp(a0, _mm512_loadu_si512(w + k), _mm512_loadu_si512(x + k));
    a1 = dp(a1, _mm512_loadu_si512(w + k + 32), _mm512_loadu_si512(x + k + 32));
  }
  for (; k < K; k += 32) {
    const int r = K - k;
    const __mmask32 m = r >= 32 ? 0xffffffffu : ((1u << r) - 1u);
    a0 = dp(a0, _mm512_maskz_loadu_epi16(m, w + k), _mm512_maskz_loadu_epi16(m, x + k));
  }
  return _mm512_reduce_add_ps(_mm512_add_ps(a0, a1));
}

// nvfp4 row: codes (K/2 bytes, element 2j in the low nibble of byte j), e4m3
// scales per 16 elements; the row global is applied by the caller.  K % 32 == 0.
OES_AVX512 float dot_nvfp4(const uint8_t *c, const uint8_t *sc, const uint16_t *x, int K, const Tables &t) {
  const __m512i lut = _mm512_load_si512(t.e2m1);
  const __m512i nib = _mm512_set1_epi32(0xf);
  __m512 acc = _mm512_setzero_ps();
  for (int g = 0; g < K / 32; ++g) {
    const __m512i d = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i *>(c + 16 * g)));
    const __m512i lo = _mm512_and_si512(d, nib);
    const __m512i hi = _mm512_and_si512(_mm512_srli_epi32(d, 4), nib);
    const __m512i idx = _mm512_or_si512(lo, _mm512_slli_epi32(hi, 16));  // words in element order
    const __m512i wv = _mm512_permutexvar_epi16(idx, lut);
    const __m512 p = dp(_mm512_setzero_ps(), wv, _mm512_loadu_si512(x + 32 * g));
    // lanes 0..7 sum elements 0..15 (first scale), lanes 8..15 elements 16..31
    const __m512 s = _mm512_mask_blend_ps(0xff00, _mm512_set1_ps(t.e4m3[sc[2 * g]]),
                                          _mm512_set1_ps(t.e4m3[sc[2 * g + 1]]));
    acc = _mm512_fmadd_ps(p, s, acc);
  }
  return _mm512_reduce_add_ps(acc);
}

// up to 16 e4m3 bytes (mask mk) -> 16 floats (OCP e4m3: bias 7, subnormals
// m * 2^-9, S.1111.111 NaN); masked-off bytes read as 0
OES_AVX512 __m512 e4m3x16(const uint8_t *b, __mmask16 mk) {
  const __m512i d = _mm512_cvtepu8_epi32(_mm_maskz_loadu_epi8(mk, b));
  const __m512i sign = _mm512_slli_epi32(_mm512_and_si512(d, _mm512_set1_epi32(0x80)), 24);
  const __m512i e = _mm512_and_si512(_mm512_srli_epi32(d, 3), _mm512_set1_epi32(15));
  const __m512i m = _mm512_and_si512(d, _mm512_set1_epi32(7));
  const __m512i normal = _mm512_or_si512(_mm512_slli_epi32(_mm512_add_epi32(e, _mm512_set1_epi32(120)), 23),
                                         _mm512_slli_epi32(m, 20));
  const __m512i sub = _mm512_castps_si512(_mm512_mul_ps(_mm512_cvtepi32_ps(m), _mm512_set1_ps(1.f / 512.f)));
  __m512i mag = _mm512_mask_blend_epi32(_mm512_cmpeq_epi32_mask(e, _mm512_setzero_si512()), normal, sub);
  mag = _mm512_mask_blend_epi32(_mm512_cmpeq_epi32_mask(_mm512_and_si512(d, _mm512_set1_epi32(0x7f)),
                                                        _mm512_set1_epi32(0x7f)),
                                mag, _mm512_set1_epi32(0x7fc00000));
  return _mm512_castsi512_ps(_mm512_or_si512(mag, sign));
}

// nvfp4 row (K % 64 == 0) against the operand split into even (xe) and odd (xo)
// elements, 64 elements per step: the 32 code bytes widen to 32 words whose low
// nibbles are the even elements and high nibbles the odd ones, so two table
// lookups and two chained vdpbf16ps cover the step; output lane i sums elements
// 4i..4i+3 of the step, scale block 4 * step + i / 4.
OES_AVX512 float dot_nvfp4_eo(const uint8_t *c, const uint8_t *sc, const uint16_t *xe, const uint16_t *xo, int K,
                              const Tables &t) {
  const __m512i lut = _mm512_load_si512(t.e2m1);
  const __m512i nib = _mm512_set1_epi16(0xf);
  const __m512i rep0 = _mm512_setr_epi32(0, 0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3);
  __m512 acc = _mm512_setzero_ps();
  __m512 s16 = _mm512_setzero_ps();
  for (int g = 0; g < K / 64; ++g) {
    if ((g & 3) == 0) {  // the scales of this step and the next three (masked at the row's end)
      const int avail = K / 16 - 4 * g;
      s16 = e4m3x16(sc + 4 * g, avail >= 16 ? (__mmask16)0xffff : (__mmask16)((1u << avail) - 1u));
    }
    const __m512i w = _mm512_cvtepu8_epi16(_mm256_loadu_si256(reinterpret_cast<const __m256i *>(c + 32 * g)));
    const __m512i lo = _mm512_and_si512(w, nib);
    const __m512i hi = _mm512_srli_epi16(w, 4);
    __m512 p = dp(_mm512_setzero_ps(), _mm512_permutexvar_epi16(lo, lut), _mm512_loadu_si512(xe + 32 * g));
    p = dp(p, _mm512_permutexvar_epi16(hi, lut), _mm512_loadu_si512(xo + 32 * g));
    const __m512i idx = _mm512_add_epi32(rep0, _mm512_set1_epi32(4 * (g & 3)));
    acc = _mm512_fmadd_ps(p, _mm512_permutexvar_ps(idx, s16), acc);
  }
  return _mm512_reduce_add_ps(acc);
}

// GGUF Q4_0 row: 16 code bytes per 32-element block (byte j: element j low
// nibble, element j + 16 high nibble), fp16 d per block.  K % 32 == 0.
OES_AVX512 float dot_q4_0(const uint8_t *c, const uint16_t *d, const uint16_t *x, int K, const Tables &t) {
  const __m512i lut = _mm512_load_si512(t.q4);
  const __m256i nib = _mm256_set1_epi16(0xf);
  __m512 acc = _mm512_setzero_ps();
  for (int g = 0; g < K / 32; ++g) {
    const __m256i b = _mm256_cvtepu8_epi16(_mm_loadu_si128(reinterpret_cast<const __m128i *>(c + 16 * g)));
    const __m256i lo = _mm256_and_si256(b, nib);
    const __m256i hi = _mm256_srli_epi16(b, 4);
    const __m512i idx = _mm512_inserti64x4(_mm512_castsi256_si512(lo), hi, 1);
    const __m512i wv = _mm512_permutexvar_epi16(idx, lut);
    const __m512 p = dp(_mm512_setzero_ps(), wv, _mm512_loadu_si512(x + 32 * g));
    acc = _mm512_fmadd_ps(p, _mm512_set1_ps(fp16_value(d[g])), acc);
  }
  return _mm512_reduce_add_ps(acc);
}

// Sum of the 64-bit words of a buffer (the DRAM read probe's loop).
OES_AVX512 uint64_t read_sum(const uint8_t *p, int64_t bytes) {
  __m512i a0 = _mm512_setzero_si512(), a1 = a0, a2 = a0, a3 = a0;
  int64_t i = 0;
  for (; i + 256 <= bytes; i += 256) {
    a0 = _mm512_xor_si512(a0, _mm512_loadu_si512(p + i));
    a1 = _mm512_xor_si512(a1, _mm512_loadu_si512(p + i + 64));
    a2 = _mm512_xor_si512(a2, _mm512_loadu_si512(p + i + 128));
    a3 = _mm512_xor_si512(a3, _mm512_loadu_si512(p + i + 192));
  }
  uint64_t r = (uint64_t)_mm512_reduce_add_epi64(_mm512_xor_si512(_mm512_xor_si512(a0, a1), _mm512_xor_si512(a2, a3)));
  for (; i < bytes; ++i) r += p[i];
  return r;
}

bool host_supported() {
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
         __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512bf16") &&
         __builtin_cpu_supports("f16c") && __builtin_cpu_supports("fma");
}

bool has_cpu_path(int fmt) { return fmt == OES_BF16 || fmt == OES_NVFP4 || fmt == OES_Q4_0; }

// CPUs this process may use: its affinity mask, capped by a cgroup v2 CPU quota
// ("quota period" in /sys/fs/cgroup/cpu.max; "max" means none).
int usable_cpus() {
  int n;
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    n = CPU_COUNT(&set);
  } else {
    const unsigned h = std::thread::hardware_concurrency();
    n = h ? (int)h : 1;
  }
  if (FILE *f = fopen("/sys/fs/cgroup/cpu.max", "r")) {
    char quota[32] = {0};
    long long period = 0;
    if (fscanf(f, "%31s %lld", quota, &period) == 2 && strcmp(quota, "max") != 0 && period > 0) {
      const long long q = atoll(quota);
      if (q > 0) n = std::min<long long>(n, std::max<long long>(1, q / period));
    }
    fclose(f);
  }
  return n < 1 ? 1 : n;
}

// Default pool size: three quarters of the usable CPUs.  The executor is bound
// by DRAM bandwidth well before that many threads, and the rest is left to the
// caller's other threads (runtime, Python): with every CPU of a CPU quota busy,
// those push the process over its quota and it is throttled for the rest of
// the period (measured on a 16-CPU quota: 16 threads 4 ms per call, 12 threads
// 0.53 ms).
int default_threads() { return std::max(1, usable_cpus() * 3 / 4); }

}  // namespace

struct oes_cpu_moe {
  oes_schema sc;
  std::vector<const uint8_t *> src;  // [bank * L + layer]
  std::unique_ptr<Pool> pool;
  Tables tab;
  std::vector<uint16_t> h;           // [pairs, I] bf16 (nvfp4: even elements, then odd)
  std::vector<uint16_t> xeo;         // nvfp4: x split into even and odd elements
  std::vector<int32_t> pt, pj;       // CPU pairs in (t, j) order
};

namespace {

// One expert's matrix rows for the dot kernels.
struct MatView {
  const uint8_t *codes;  // row r at codes + r * row_bytes
  int64_t row_bytes;
  const uint8_t *scale;  // nvfp4: e4m3 [rows][K/16]; q4_0: fp16 [rows][K/32]
  int64_t scale_ld;      // bytes per row of scale
  const uint8_t *glob;   // nvfp4: fp16 [rows]
  int K;
};

MatView mat_view(const oes_cpu_moe *m, int layer, int e, bool down) {
  const oes_schema &sc = m->sc;
  const int L = sc.num_layers;
  auto row = [&](int b) { return m->src[(size_t)b * L + layer] + (int64_t)e * sc.bank[b].row_bytes; };
  MatView v = {};
  v.K = down ? sc.inter : sc.hidden;
  if (sc.format == OES_BF16) {
    const int b = down ? 1 : 0;
    v.codes = row(b);
    v.row_bytes = 2ll * v.K;
  } else if (sc.format == OES_NVFP4) {
    const int b = down ? 3 : 0;
    v.codes = row(b);
    v.row_bytes = v.K / 2;
    v.scale = row(b + 1);
    v.scale_ld = v.K / 16;
    v.glob = row(b + 2);
  } else {  // Q4_0
    const int b = down ? 2 : 0;
    v.codes = row(b);
    v.row_bytes = v.K / 2;
    v.scale = row(b + 1);
    v.scale_ld = (v.K / 32) * 2;
  }
  return v;
}

// x: the operand in element order, or for nvfp4 with eo set its even elements
// followed by its odd ones (K % 64 == 0)
OES_AVX512 float row_dot(int fmt, const MatView &v, int r, const uint16_t *x, const Tables &t, bool eo) {
  const uint8_t *c = v.codes + (int64_t)r * v.row_bytes;
  if (fmt == OES_BF16) return dot_bf16(reinterpret_cast<const uint16_t *>(c), x, v.K);
  if (fmt == OES_NVFP4) {
    const uint8_t *sc = v.scale + (int64_t)r * v.scale_ld;
    const float s = eo ? dot_nvfp4_eo(c, sc, x, x + v.K / 2, v.K, t) : dot_nvfp4(c, sc, x, v.K, t);
    return s * fp16_value(reinterpret_cast<const uint16_t *>(v.glob)[r]);
  }
  return dot_q4_0(c, reinterpret_cast<const uint16_t *>(v.scale + (int64_t)r * v.scale_ld), x, v.K, t);
}

}  // namespace

namespace oes {
const oes_schema *cpu_moe_schema(const oes_cpu_moe *m) { return &m->sc; }
}  // namespace oes

extern "C" oes_status oes_cpu_moe_create(const oes_schema *sc, int32_t threads, oes_cpu_moe **out) {
  if (!out) return fail(OES_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!sc) return fail(OES_ERR_ARG, "schema is NULL");
  oes_schema ref;
  if (oes_schema_make(sc->format, sc->num_layers, sc->num_experts, sc->hidden, sc->inter, &ref) != OES_OK)
    return OES_ERR_ARG;  // message left by oes_schema_make
  if (memcmp(&ref, sc, sizeof(ref)) != 0) return fail(OES_ERR_ARG, "schema was modified after oes_schema_make");
  if (!has_cpu_path(sc->format))
    return fail(OES_ERR_UNSUPPORTED, "format %d has no CPU MoE path (bf16, nvfp4 and q4_0 have one)", sc->format);
  if (!host_supported()) return fail(OES_ERR_UNSUPPORTED, "the host CPU lacks AVX-512 F/BW/VL/BF16 or F16C");
  if (threads < 0 || threads > 1024) return fail(OES_ERR_ARG, "threads %d outside [0, 1024]", threads);
  const int n = threads ? threads : default_threads();
  oes_cpu_moe *m = new oes_cpu_moe();
  m->sc = *sc;
  m->src.assign((size_t)sc->num_banks * sc->num_layers, nullptr);
  for (int c = 0; c < 32; ++c) {
    m->tab.e2m1[c] = bf16_rne(e2m1_value((uint8_t)(c & 15)));
    m->tab.q4[c] = bf16_rne((float)((c & 15) - 8));
  }
  for (int c = 0; c < 256; ++c) m->tab.e4m3[c] = e4m3_value((uint8_t)c);
  m->pool.reset(new Pool(n));
  *out = m;
  return OES_OK;
}

extern "C" oes_status oes_cpu_moe_destroy(oes_cpu_moe *m) {
  delete m;
  return OES_OK;
}

extern "C" oes_status oes_cpu_moe_threads(const oes_cpu_moe *m, int32_t *threads) {
  if (!m || !threads) return fail(OES_ERR_ARG, "NULL argument");
  *threads = m->pool->size();
  return OES_OK;
}

extern "C" oes_status oes_cpu_moe_set_source(oes_cpu_moe *m, int32_t bank, int32_t layer, const void *host,
                                             int64_t bytes) {
  if (!m) return fail(OES_ERR_ARG, "executor is NULL");
  const oes_schema &sc = m->sc;
  if (bank < 0 || bank >= sc.num_banks) return fail(OES_ERR_ARG, "bank %d out of range", bank);
  if (layer < 0 || layer >= sc.num_layers) return fail(OES_ERR_ARG, "layer %d out of range", layer);
  if (!host) return fail(OES_ERR_ARG, "host is NULL");
  const int64_t want = (int64_t)sc.num_experts * sc.bank[bank].row_bytes;
  if (bytes != want) return fail(OES_ERR_ARG, "bank %d: %lld bytes, expected %lld", bank, (long long)bytes, (long long)want);
  m->src[(size_t)bank * sc.num_layers + layer] = static_cast<const uint8_t *>(host);
  // Touch every 4 KiB page once: the first CPU read of pinned memory that only
  // the GPU has written maps its pages (measured: 390 ms for 1.15 GB on first
  // touch, 2.8 ms for the same walk afterwards); doing it here keeps that cost
  // out of the steps.
  const volatile uint8_t *p = static_cast<const volatile uint8_t *>(host);
  std::vector<uint32_t> sink(m->pool->size(), 0);
  m->pool->run([&](int tid, int nt) {
    const int64_t pages = (bytes + 4095) / 4096;
    uint32_t acc = 0;
    for (int64_t i = pages * tid / nt; i < pages * (tid + 1) / nt; ++i) acc += p[i * 4096];
    sink[tid] = acc;
  });
  return OES_OK;
}

extern "C" oes_status oes_cpu_moe_run(oes_cpu_moe *m, int32_t layer, const void *x_bf16, const int32_t *ids,
                                      const int32_t *slot_ids, const float *w, int32_t n, int32_t k, float *y) {
  if (!m) return fail(OES_ERR_ARG, "executor is NULL");
  const oes_schema &sc = m->sc;
  if (n < 0 || k < 1 || k > 64) return fail(OES_ERR_ARG, "n = %d, k = %d", n, k);
  if (n == 0) return OES_OK;
  if (!x_bf16 || !ids || !slot_ids || !w || !y) return fail(OES_ERR_ARG, "NULL buffer");
  if (layer < 0 || layer >= sc.num_layers) return fail(OES_ERR_ARG, "layer %d out of range", layer);
  const int H = sc.hidden, I = sc.inter, E = sc.num_experts;
  m->pt.clear();
  m->pj.clear();
  for (int t = 0; t < n; ++t)
    for (int j = 0; j < k; ++j) {
      if (slot_ids[t * k + j] >= 0) continue;
      const int e = ids[t * k + j];
      if (e < 0 || e >= E) return fail(OES_ERR_ARG, "ids[%d][%d] = %d outside [0, %d)", t, j, e, E);
      m->pt.push_back(t);
      m->pj.push_back(j);
    }
  const int P = (int)m->pt.size();
  if (P) {
    for (int b = 0; b < sc.num_banks; ++b)
      if (!m->src[(size_t)b * sc.num_layers + layer])
        return fail(OES_ERR_ARG, "bank %d has no source for layer %d", b, layer);
  }
  m->h.resize((size_t)P * I);
  const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
  const int fmt = sc.format;
  // nvfp4 rows of a multiple of 64 elements take their operand as even elements
  // then odd ones: x is split here, h is written split by pass 1
  const bool eo_gu = fmt == OES_NVFP4 && H % 64 == 0, eo_dn = fmt == OES_NVFP4 && I % 64 == 0;
  if (P && eo_gu) {
    m->xeo.resize((size_t)n * H);
    for (int t = 0; t < n; ++t)
      for (int j = 0; j < H / 2; ++j) {
        m->xeo[(size_t)t * H + j] = x[(int64_t)t * H + 2 * j];
        m->xeo[(size_t)t * H + H / 2 + j] = x[(int64_t)t * H + 2 * j + 1];
      }
    x = m->xeo.data();
  }
  const Tables &tab = m->tab;
  uint16_t *hb = m->h.data();
  const int32_t *pt = m->pt.data(), *pj = m->pj.data();

  if (P) {
    // pass 1: gate_up + SiLU * up over the flattened (pair, feature) space
    const int64_t items = (int64_t)P * I;
    m->pool->run([&](int tid, int nt) {
      const int64_t lo = items * tid / nt, hi = items * (tid + 1) / nt;
      int cur = -1;
      MatView v = {};
      for (int64_t it = lo; it < hi; ++it) {
        const int p = (int)(it / I), r = (int)(it % I);
        if (p != cur) {
          v = mat_view(m, layer, ids[pt[p] * k + pj[p]], false);
          cur = p;
        }
        const uint16_t *xt = x + (int64_t)pt[p] * H;
        const float g = row_dot(fmt, v, r, xt, tab, eo_gu);
        const float u = row_dot(fmt, v, r + I, xt, tab, eo_gu);
        const int64_t at = (int64_t)p * I + (eo_dn ? (r & 1) * (I / 2) + (r >> 1) : r);
        hb[at] = bf16_rne(g / (1.f + expf(-g)) * u);
      }
    });
  }
  // pass 2: down + combine over output rows (tokens without CPU pairs get 0)
  m->pool->run([&](int tid, int nt) {
    const int lo = (int)((int64_t)H * tid / nt), hi = (int)((int64_t)H * (tid + 1) / nt);
    for (int t = 0; t < n; ++t)
      for (int r = lo; r < hi; ++r) y[(int64_t)t * H + r] = 0.f;
    for (int p = 0; p < P; ++p) {
      const MatView v = mat_view(m, layer, ids[pt[p] * k + pj[p]], true);
      const float wt = w[pt[p] * k + pj[p]];
      float *yt = y + (int64_t)pt[p] * H;
      const uint16_t *hp = hb + (int64_t)p * I;
      for (int r = lo; r < hi; ++r) yt[r] += wt * row_dot(fmt, v, r, hp, tab, eo_dn);
    }
  });
  return OES_OK;
}

extern "C" oes_status oes_cpu_moe_probe_read(oes_cpu_moe *m, const void *buf, int64_t bytes, double *ms) {
  if (!m || !buf || !ms) return fail(OES_ERR_ARG, "NULL argument");
  if (bytes <= 0) return fail(OES_ERR_ARG, "bytes must be positive");
  const uint8_t *p = static_cast<const uint8_t *>(buf);
  std::vector<uint64_t> part(m->pool->size(), 0);
  const auto t0 = std::chrono::steady_clock::now();
  m->pool->run([&](int tid, int nt) {
    const int64_t lo = bytes * tid / nt / 64 * 64, hi = tid + 1 == nt ? bytes : bytes * (tid + 1) / nt / 64 * 64;
    part[tid] = read_sum(p + lo, hi - lo);
  });
  const auto t1 = std::chrono::steady_clock::now();
  uint64_t s = 0;
  for (uint64_t v : part) s += v;
  if (s == 0x5a5a5a5a5a5a5a5aull) fprintf(stderr, "%llu\n", (unsigned long long)s);  // keeps the reads alive
  *ms = std::chrono::duration<double, std::milli>(t1 - t0).count();
  return OES_OK;
}

extern "C" oes_status oes_hybrid_decide(int32_t format, double cpu_gbps, double pcie_gbps, double threshold,
                                        int32_t *hybrid, double *fetch_fraction) {
  if (!hybrid || !fetch_fraction) return fail(OES_ERR_ARG, "NULL argument");
  if (!(cpu_gbps >= 0) || !(pcie_gbps > 0) || !(threshold > 0))
    return fail(OES_ERR_ARG, "bandwidths must be >= 0 (pcie > 0) and the threshold > 0");
  *hybrid = has_cpu_path(format) && cpu_gbps > threshold * pcie_gbps ? 1 : 0;
  *fetch_fraction = cpu_gbps <= pcie_gbps ? 1.0 : pcie_gbps / cpu_gbps;
  return OES_OK;
}
