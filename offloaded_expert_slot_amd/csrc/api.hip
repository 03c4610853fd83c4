// Host side of liboes.so: argument checking, ownership, and launch of the HIP kernels.
//
// Every exported function validates its arguments before touching the GPU,
// returns an oes_status and leaves a message in a thread-local string on
// error.  Step calls only enqueue work on the caller's stream.

#include <stdarg.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "oes_internal.h"

using namespace oes;

namespace {

oes_status fail(oes_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
oes_status fail(oes_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return set_error(st, buf);
}

}  // namespace

namespace {

oes_status hip_fail(hipError_t e, const char *what) {
  (void)hipGetLastError();  // clear the runtime's sticky last-error slot
  return fail(OES_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr)                                   \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return hip_fail(e_, #expr);   \
  } while (0)

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Scoped device switch.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};


// Returns the device-readable address of pinned host memory, or nullptr.
const void *device_view_of_host(const void *host) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost) return nullptr;
  void *dev = nullptr;
  if (hipHostGetDevicePointer(&dev, const_cast<void *>(host), 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return dev;
}

oes_status check_schema(const oes_schema *sc) {
  if (!sc) return fail(OES_ERR_ARG, "schema is NULL");
  oes_schema tmp;
  oes_status st = oes_schema_make(sc->format, sc->num_layers, sc->num_experts, sc->hidden,
                                  sc->inter, &tmp);
  if (st != OES_OK) return st;
  if (memcmp(&tmp, sc, sizeof(tmp)) != 0)
    return fail(OES_ERR_ARG, "schema was modified after oes_schema_make");
  return OES_OK;
}

// Bank sources: per (bank, layer) the caller's host address and its device view.
struct Sources {
  int nb = 0, L = 0;
  std::vector<const void *> host;  // [nb * L]
  std::vector<uint64_t> dev;       // [nb * L], 0 = none
  uint64_t *d_table = nullptr;     // device copy of `dev`, laid out [nb][L]

  oes_status init(int banks, int layers) {
    nb = banks;
    L = layers;
    host.assign((size_t)nb * L, nullptr);
    dev.assign((size_t)nb * L, 0);
    hipError_t e = hipMalloc(&d_table, sizeof(uint64_t) * nb * L);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(source table)");
    e = hipMemcpy(d_table, dev.data(), sizeof(uint64_t) * nb * L, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(source table)");
    return OES_OK;
  }
  void release() {
    if (d_table) (void)hipFree(d_table);
    d_table = nullptr;
  }
  oes_status set(const oes_schema &sc, int bank, int layer, const void *h, int64_t bytes) {
    if (bank < 0 || bank >= nb) return fail(OES_ERR_ARG, "bank %d outside [0, %d)", bank, nb);
    if (layer < 0 || layer >= L) return fail(OES_ERR_ARG, "layer %d outside [0, %d)", layer, L);
    if (!h) return fail(OES_ERR_ARG, "host pointer is NULL");
    if (reinterpret_cast<uintptr_t>(h) % 16)
      return fail(OES_ERR_ARG, "host bank must be 16-byte aligned");
    int64_t want = (int64_t)sc.num_experts * sc.bank[bank].row_bytes;
    if (bytes != want)
      return fail(OES_ERR_ARG, "bank %d layer %d: %lld bytes, expected E*row_bytes = %lld", bank,
                  layer, (long long)bytes, (long long)want);
    const void *d = device_view_of_host(h);
    if (!d) return fail(OES_ERR_ARG, "bank %d layer %d: host memory is not pinned (hipHostMalloc)", bank, layer);
    // the whole range must be pinned too
    const void *d_end = device_view_of_host(static_cast<const uint8_t *>(h) + bytes - 1);
    if (!d_end || static_cast<const uint8_t *>(d_end) != static_cast<const uint8_t *>(d) + bytes - 1)
      return fail(OES_ERR_ARG, "bank %d layer %d: range is not one pinned allocation", bank, layer);
    host[(size_t)bank * L + layer] = h;
    dev[(size_t)bank * L + layer] = reinterpret_cast<uint64_t>(d);
    hipError_t e = hipMemcpy(d_table + (size_t)bank * L + layer, &dev[(size_t)bank * L + layer],
                             sizeof(uint64_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(source entry)");
    return OES_OK;
  }
};

}  // namespace

// ============================================================================ cache object
struct oes_cache {
  oes_schema sc;
  int S = 0, device = 0, maxM = 0, Spad = 0;
  uint8_t *slot_bank[OES_MAX_BANKS] = {};
  // one device block: owner | stamp | ctl | miss_slot | miss_id | aux_slot | aux_id
  uint8_t *dblock = nullptr;
  int64_t *owner = nullptr;
  uint64_t *stamp = nullptr;
  Ctl *ctl = nullptr;
  int32_t *miss_slot = nullptr;
  int64_t *miss_id = nullptr;
  int32_t *aux_slot = nullptr;
  int64_t *aux_id = nullptr;
  Sources src;
  // pinned staging for host<->device transfers of the table
  uint8_t *staging = nullptr;
  int64_t staging_bytes = 0;
  hipEvent_t staging_done = nullptr;
  int fused_copy = 1, copy_mode = OES_COPY_ZERO, copy_blocks = 0, ffn_path = OES_FFN_AUTO;
  uint8_t *snap = nullptr;  // device snapshot: owner | stamp | clock
  bool has_snap = false;
  hipEvent_t hybrid_ev = nullptr;  // hybrid step: the step's ids have reached the host
};

struct oes_layers {
  oes_schema sc;
  int depth = 2, device = 0;
  std::vector<uint8_t *> buf;   // [depth * nb]
  Sources src;
  std::vector<hipEvent_t> ready, released;
  std::vector<int> resident;   // layer held by each buffer (-1 none)
};

// ============================================================================ cache lifecycle
// The slot table of S slots in one device block (owner | stamp | ctl | miss list |
// load list) plus its pinned staging buffer.
struct TableBufs {
  uint8_t *dblock = nullptr;
  int64_t *owner = nullptr;
  uint64_t *stamp = nullptr;
  Ctl *ctl = nullptr;
  int32_t *miss_slot = nullptr;
  int64_t *miss_id = nullptr;
  int32_t *aux_slot = nullptr;
  int64_t *aux_id = nullptr;
  uint8_t *staging = nullptr;
  int64_t staging_bytes = 0;
};

static void table_free(TableBufs *t) {
  if (t->dblock) (void)hipFree(t->dblock);
  if (t->staging) (void)hipHostFree(t->staging);
  *t = TableBufs();
}

static oes_status table_alloc(int64_t S, TableBufs *t) {
  *t = TableBufs();
  int64_t off = 0;
  const int64_t o_owner = off; off = round_up(off + 8 * S, 256);
  const int64_t o_stamp = off; off = round_up(off + 8 * S, 256);
  const int64_t o_ctl = off;   off = round_up(off + (int64_t)sizeof(Ctl), 256);
  const int64_t o_ms = off;    off = round_up(off + 4 * S, 256);
  const int64_t o_mi = off;    off = round_up(off + 8 * S, 256);
  const int64_t o_as = off;    off = round_up(off + 4 * S, 256);
  const int64_t o_ai = off;    off = round_up(off + 8 * S, 256);
  hipError_t e = hipMalloc(&t->dblock, off);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    t->dblock = nullptr;
    return fail(OES_ERR_NOMEM, "hipMalloc of the slot table failed");
  }
  t->owner = reinterpret_cast<int64_t *>(t->dblock + o_owner);
  t->stamp = reinterpret_cast<uint64_t *>(t->dblock + o_stamp);
  t->ctl = reinterpret_cast<Ctl *>(t->dblock + o_ctl);
  t->miss_slot = reinterpret_cast<int32_t *>(t->dblock + o_ms);
  t->miss_id = reinterpret_cast<int64_t *>(t->dblock + o_mi);
  t->aux_slot = reinterpret_cast<int32_t *>(t->dblock + o_as);
  t->aux_id = reinterpret_cast<int64_t *>(t->dblock + o_ai);
  t->staging_bytes = round_up(16 * S + (int64_t)sizeof(Ctl) + 12 * S + 64, 256);
  e = hipHostMalloc(reinterpret_cast<void **>(&t->staging), t->staging_bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    t->staging = nullptr;
    table_free(t);
    return fail(OES_ERR_NOMEM, "hipHostMalloc of the staging buffer failed");
  }
  return OES_OK;
}

static void table_adopt(oes_cache *c, const TableBufs &t) {
  c->dblock = t.dblock;
  c->owner = t.owner;
  c->stamp = t.stamp;
  c->ctl = t.ctl;
  c->miss_slot = t.miss_slot;
  c->miss_id = t.miss_id;
  c->aux_slot = t.aux_slot;
  c->aux_id = t.aux_id;
  c->staging = t.staging;
  c->staging_bytes = t.staging_bytes;
}

static int pad_pow2(int S) {
  int p = 2;
  while (p < S) p <<= 1;
  return p;
}

static void cache_free(oes_cache *c) {
  for (int b = 0; b < OES_MAX_BANKS; ++b)
    if (c->slot_bank[b]) (void)hipFree(c->slot_bank[b]);
  if (c->dblock) (void)hipFree(c->dblock);
  if (c->snap) (void)hipFree(c->snap);
  if (c->staging) (void)hipHostFree(c->staging);
  if (c->staging_done) (void)hipEventDestroy(c->staging_done);
  if (c->hybrid_ev) (void)hipEventDestroy(c->hybrid_ev);
  c->src.release();
  delete c;
}

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

extern "C" oes_status oes_cache_create(const oes_schema *sc, int32_t num_slots, int32_t device,
                                       oes_cache **out) {
  if (!out) return fail(OES_ERR_ARG, "out is NULL");
  *out = nullptr;
  oes_status st = check_schema(sc);
  if (st != OES_OK) return st;
  if (num_slots < 1 || num_slots > OES_MAX_SLOTS)
    return fail(OES_ERR_ARG, "num_slots %d outside [1, %d]", num_slots, OES_MAX_SLOTS);
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev) return fail(OES_ERR_ARG, "device %d outside [0, %d)", device, ndev);
  DeviceGuard g(device);
  if (!g.ok) return fail(OES_ERR_HIP, "hipSetDevice(%d) failed", device);

  oes_cache *c = new oes_cache();
  c->sc = *sc;
  c->S = num_slots;
  c->device = device;
  c->maxM = std::min(num_slots, sc->num_experts);
  c->Spad = pad_pow2(num_slots);
  for (int b = 0; b < sc->num_banks; ++b) {
    e = hipMalloc(&c->slot_bank[b], (size_t)num_slots * sc->bank[b].row_bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      cache_free(c);
      return fail(OES_ERR_NOMEM, "hipMalloc of slot bank %s (%lld bytes) failed", sc->bank[b].name,
                  (long long)num_slots * sc->bank[b].row_bytes);
    }
  }
  const int64_t S = num_slots;
  {
    TableBufs t;
    st = table_alloc(S, &t);
    if (st != OES_OK) {
      cache_free(c);
      return st;
    }
    table_adopt(c, t);
  }
  e = hipEventCreateWithFlags(&c->staging_done, hipEventDisableTiming);
  if (e != hipSuccess) { cache_free(c); return hip_fail(e, "hipEventCreate"); }
  st = c->src.init(sc->num_banks, sc->num_layers);
  if (st != OES_OK) { cache_free(c); return st; }
  // initial state: all empty, stamps 0, clock 0, no error
  std::vector<int64_t> own(S, -1);
  e = hipMemcpy(c->owner, own.data(), 8 * S, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(c->stamp, 0, 8 * S);
  Ctl ctl0;
  memset(&ctl0, 0, sizeof(ctl0));
  ctl0.step_ok = 1;  // no failed step yet: copy / FFN run
  if (e == hipSuccess) e = hipMemcpy(c->ctl, &ctl0, sizeof(Ctl), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) { cache_free(c); return hip_fail(e, "initialising the slot table"); }
  c->fused_copy = env_int("OES_FUSED_COPY", 1) ? 1 : 0;
  const char *mode = getenv("OES_COPY_MODE");
  c->copy_mode = (mode && strcmp(mode, "sdma") == 0) ? OES_COPY_SDMA : OES_COPY_ZERO;
  *out = c;
  return OES_OK;
}

extern "C" oes_status oes_cache_destroy(oes_cache *c) {
  if (!c) return OES_OK;
  DeviceGuard g(c->device);
  (void)hipDeviceSynchronize();
  cache_free(c);
  return OES_OK;
}

extern "C" oes_status oes_cache_set_source(oes_cache *c, int32_t bank, int32_t layer, const void *host,
                                           int64_t bytes) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  DeviceGuard g(c->device);
  return c->src.set(c->sc, bank, layer, host, bytes);
}

extern "C" oes_status oes_cache_set_option(oes_cache *c, int32_t option, int64_t value) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  switch (option) {
    case OES_OPT_FUSED_COPY: c->fused_copy = value ? 1 : 0; return OES_OK;
    case OES_OPT_COPY_MODE:
      if (value != OES_COPY_ZERO && value != OES_COPY_SDMA) return fail(OES_ERR_ARG, "bad copy mode");
      c->copy_mode = (int)value;
      return OES_OK;
    case OES_OPT_COPY_BLOCKS:
      if (value < 0 || value > 65536) return fail(OES_ERR_ARG, "copy blocks outside [0, 65536]");
      c->copy_blocks = (int)value;
      return OES_OK;
    case OES_OPT_FFN_PATH:
      if (value != OES_FFN_AUTO && value != OES_FFN_PER_PAIR && value != OES_FFN_GROUPED)
        return fail(OES_ERR_ARG, "bad FFN path");
      c->ffn_path = (int)value;
      return OES_OK;
    default: return fail(OES_ERR_ARG, "unknown option %d", option);
  }
}

extern "C" oes_status oes_cache_info(const oes_cache *c, int32_t *num_slots, oes_schema *schema) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (num_slots) *num_slots = c->S;
  if (schema) *schema = c->sc;
  return OES_OK;
}

extern "C" oes_status oes_cache_slot_bank(const oes_cache *c, int32_t bank, void **dev_base,
                                          int64_t *row_bytes) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (bank < 0 || bank >= c->sc.num_banks) return fail(OES_ERR_ARG, "bank %d out of range", bank);
  if (dev_base) *dev_base = c->slot_bank[bank];
  if (row_bytes) *row_bytes = c->sc.bank[bank].row_bytes;
  return OES_OK;
}

// Waits until the previous transfer through the staging buffer has finished.
static oes_status staging_acquire(oes_cache *c) {
  hipError_t e = hipEventSynchronize(c->staging_done);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
  return OES_OK;
}

extern "C" oes_status oes_cache_set_state(oes_cache *c, const int64_t *owner, const uint64_t *stamp,
                                          uint64_t clock, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (!owner || !stamp) return fail(OES_ERR_ARG, "owner and stamp must not be NULL");
  const int S = c->S;
  if (clock >= (1ull << 62)) return fail(OES_ERR_ARG, "clock >= 2^62");
  std::vector<int64_t> seen;
  seen.reserve(S);
  for (int s = 0; s < S; ++s) {
    if (owner[s] < -1 || owner[s] >= (1ll << 50)) return fail(OES_ERR_ARG, "owner[%d] = %lld out of range", s, (long long)owner[s]);
    if (stamp[s] >= (1ull << 62)) return fail(OES_ERR_ARG, "stamp[%d] >= 2^62", s);
    if (owner[s] >= 0) seen.push_back(owner[s]);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(OES_ERR_ARG, "an owner id appears in two slots");
  DeviceGuard g(c->device);
  oes_status st = staging_acquire(c);
  if (st != OES_OK) return st;
  uint8_t *p = c->staging;
  memcpy(p, owner, 8 * (size_t)S);
  memcpy(p + 8 * (size_t)S, stamp, 8 * (size_t)S);
  hipStream_t s = as_stream(stream);
  // the counters are kept: only clock / err / step_ok / miss_count are written
  Ctl *hc = reinterpret_cast<Ctl *>(p + 16 * (size_t)S);
  hc->clock = clock;
  hc->err = 0;
  hc->step_ok = 1;  // a freshly set table is valid: FFN runs, copy has an empty list
  hc->miss_count = 0;
  HIP_TRY(hipMemcpyAsync(c->owner, p, 8 * (size_t)S, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->stamp, p + 8 * (size_t)S, 8 * (size_t)S, hipMemcpyHostToDevice, s));
  // clock, err, step_ok, miss_count are the first 20 bytes of Ctl
  static_assert(offsetof(Ctl, clock) == 0 && offsetof(Ctl, miss_count) == 16, "Ctl layout");
  HIP_TRY(hipMemcpyAsync(c->ctl, hc, 20, hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(c->staging_done, s));
  return OES_OK;
}

extern "C" oes_status oes_cache_snapshot(oes_cache *c, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  DeviceGuard g(c->device);
  const size_t S = (size_t)c->S;
  if (!c->snap) {
    hipError_t e = hipMalloc(&c->snap, 16 * S + 64);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(OES_ERR_NOMEM, "hipMalloc of the snapshot failed");
    }
  }
  hipStream_t s = as_stream(stream);
  HIP_TRY(hipMemcpyAsync(c->snap, c->owner, 8 * S, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->snap + 8 * S, c->stamp, 8 * S, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->snap + 16 * S, &c->ctl->clock, 8, hipMemcpyDeviceToDevice, s));
  c->has_snap = true;
  return OES_OK;
}

extern "C" oes_status oes_cache_restore(oes_cache *c, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (!c->has_snap) return fail(OES_ERR_STATE, "no snapshot taken");
  DeviceGuard g(c->device);
  const size_t S = (size_t)c->S;
  hipStream_t s = as_stream(stream);
  HIP_TRY(hipMemcpyAsync(c->owner, c->snap, 8 * S, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->stamp, c->snap + 8 * S, 8 * S, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(&c->ctl->clock, c->snap + 16 * S, 8, hipMemcpyDeviceToDevice, s));
  launch_reset_step(c->ctl, s);
  HIP_TRY(hipGetLastError());
  return OES_OK;
}

extern "C" oes_status oes_cache_get_state(oes_cache *c, int64_t *owner, uint64_t *stamp, uint64_t *clock,
                                          void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  DeviceGuard g(c->device);
  oes_status st = staging_acquire(c);
  if (st != OES_OK) return st;
  const int S = c->S;
  hipStream_t s = as_stream(stream);
  uint8_t *p = c->staging;
  HIP_TRY(hipMemcpyAsync(p, c->owner, 8 * (size_t)S, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(p + 8 * (size_t)S, c->stamp, 8 * (size_t)S, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(p + 16 * (size_t)S, c->ctl, sizeof(Ctl), hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (owner) memcpy(owner, p, 8 * (size_t)S);
  if (stamp) memcpy(stamp, p + 8 * (size_t)S, 8 * (size_t)S);
  if (clock) *clock = reinterpret_cast<Ctl *>(p + 16 * (size_t)S)->clock;
  return OES_OK;
}

static oes_status read_ctl(oes_cache *c, hipStream_t s, Ctl *out) {
  oes_status st = staging_acquire(c);
  if (st != OES_OK) return st;
  uint8_t *p = c->staging + 16 * (size_t)c->S;
  HIP_TRY(hipMemcpyAsync(p, c->ctl, sizeof(Ctl), hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  memcpy(out, p, sizeof(Ctl));
  return OES_OK;
}

extern "C" oes_status oes_cache_check(oes_cache *c, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  DeviceGuard g(c->device);
  hipStream_t s = as_stream(stream);
  Ctl ctl;
  oes_status st = read_ctl(c, s, &ctl);
  if (st != OES_OK) return st;
  if (ctl.err == OES_OK) return OES_OK;
  int32_t zero = 0;
  HIP_TRY(hipMemcpyAsync(&c->ctl->err, &zero, sizeof(zero), hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (ctl.err == OES_ERR_CAPACITY)
    return fail(OES_ERR_CAPACITY, "a step requested more distinct experts than the %d slots", c->S);
  if (ctl.err == OES_ERR_ARG)
    return fail(OES_ERR_ARG, "a step held an expert id outside [0, %d) or a layer without a source", c->sc.num_experts);
  return fail(ctl.err, "device error %d", ctl.err);
}

// Runtime resize of the slot pool (FreeToken architecture walk-through §4: VRAM
// moves between the expert cache and other uses with no restart and no weight
// reload).  Growing keeps every slot in place and appends empty ones; shrinking
// keeps the num_slots slots that come last in the remap's victim order (empty
// slots first, then least recently used: key (not empty, stamp, owner, slot)),
// packed in ascending old index.  Stamps, clock and counters are kept; the
// pending miss and load lists are cleared.  New banks and table are allocated
// and filled before the old ones are freed, so a failure leaves the cache as
// it was.
extern "C" oes_status oes_cache_resize(oes_cache *c, int32_t num_slots, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (num_slots < 1 || num_slots > OES_MAX_SLOTS)
    return fail(OES_ERR_ARG, "num_slots %d outside [1, %d]", num_slots, OES_MAX_SLOTS);
  DeviceGuard g(c->device);
  if (!g.ok) return fail(OES_ERR_HIP, "hipSetDevice(%d) failed", c->device);
  hipStream_t s = as_stream(stream);
  const int S0 = c->S, S1 = num_slots;
  // the current table; the sync also drains every step enqueued before
  oes_status st = staging_acquire(c);
  if (st != OES_OK) return st;
  HIP_TRY(hipMemcpyAsync(c->staging, c->owner, 8 * (size_t)S0, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(c->staging + 8 * (size_t)S0, c->stamp, 8 * (size_t)S0, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(c->staging + 16 * (size_t)S0, c->ctl, sizeof(Ctl), hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  std::vector<int64_t> own0(S0);
  std::vector<uint64_t> stp0(S0);
  Ctl ctl;
  memcpy(own0.data(), c->staging, 8 * (size_t)S0);
  memcpy(stp0.data(), c->staging + 8 * (size_t)S0, 8 * (size_t)S0);
  memcpy(&ctl, c->staging + 16 * (size_t)S0, sizeof(Ctl));
  if (S1 == S0) return OES_OK;

  // new slot i takes old slot src[i] (-1: new and empty)
  std::vector<int32_t> src(S1, -1);
  if (S1 > S0) {
    for (int i = 0; i < S0; ++i) src[i] = i;
  } else {
    std::vector<int32_t> order(S0);
    for (int i = 0; i < S0; ++i) order[i] = i;
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      const bool ea = own0[a] != -1, eb = own0[b] != -1;
      if (ea != eb) return !ea;
      if (stp0[a] != stp0[b]) return stp0[a] < stp0[b];
      if (own0[a] != own0[b]) return own0[a] < own0[b];
      return a < b;
    });
    std::vector<int32_t> keep(order.end() - S1, order.end());
    std::sort(keep.begin(), keep.end());
    src = keep;
  }
  std::vector<int64_t> own1(S1, -1);
  std::vector<uint64_t> stp1(S1, 0);
  for (int i = 0; i < S1; ++i)
    if (src[i] >= 0) {
      own1[i] = own0[src[i]];
      stp1[i] = stp0[src[i]];
    }

  // new table and banks
  TableBufs t;
  st = table_alloc(S1, &t);
  if (st != OES_OK) return st;
  uint8_t *nb[OES_MAX_BANKS] = {};
  auto drop_new = [&]() {
    for (int b = 0; b < OES_MAX_BANKS; ++b)
      if (nb[b]) (void)hipFree(nb[b]);
    table_free(&t);
  };
  for (int b = 0; b < c->sc.num_banks; ++b) {
    hipError_t e = hipMalloc(&nb[b], (size_t)S1 * c->sc.bank[b].row_bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      nb[b] = nullptr;
      drop_new();
      return fail(OES_ERR_NOMEM, "hipMalloc of slot bank %s (%lld bytes) failed", c->sc.bank[b].name,
                  (long long)S1 * c->sc.bank[b].row_bytes);
    }
  }
  Ctl nc = ctl;
  nc.miss_count = 0;
  nc.aux_count = 0;
  uint8_t *p = t.staging;
  memcpy(p, own1.data(), 8 * (size_t)S1);
  memcpy(p + 8 * (size_t)S1, stp1.data(), 8 * (size_t)S1);
  memcpy(p + 16 * (size_t)S1, &nc, sizeof(Ctl));
  memcpy(p + 16 * (size_t)S1 + sizeof(Ctl), src.data(), 4 * (size_t)S1);
  hipError_t e = hipMemcpyAsync(t.owner, p, 8 * (size_t)S1, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(t.stamp, p + 8 * (size_t)S1, 8 * (size_t)S1, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(t.ctl, p + 16 * (size_t)S1, sizeof(Ctl), hipMemcpyHostToDevice, s);
  // the move list goes to the new load-list area, unused until the next load_rows
  if (e == hipSuccess)
    e = hipMemcpyAsync(t.aux_slot, p + 16 * (size_t)S1 + sizeof(Ctl), 4 * (size_t)S1, hipMemcpyHostToDevice, s);
  for (int b = 0; b < c->sc.num_banks && e == hipSuccess; ++b)
    e = launch_slot_move(nb[b], c->slot_bank[b], t.aux_slot, S1, c->sc.bank[b].row_bytes, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(s);  // nothing enqueued may still use the new buffers
    drop_new();
    return hip_fail(e, "moving the slot rows");
  }

  // swap in
  for (int b = 0; b < OES_MAX_BANKS; ++b) {
    if (c->slot_bank[b]) (void)hipFree(c->slot_bank[b]);
    c->slot_bank[b] = nb[b];
  }
  (void)hipFree(c->dblock);
  (void)hipHostFree(c->staging);
  table_adopt(c, t);
  if (c->snap) (void)hipFree(c->snap);
  c->snap = nullptr;
  c->has_snap = false;
  c->S = S1;
  c->maxM = std::min(S1, c->sc.num_experts);
  c->Spad = pad_pow2(S1);
  return OES_OK;
}

extern "C" oes_status oes_cache_stats(oes_cache *c, oes_stats *out, void *stream) {
  if (!c || !out) return fail(OES_ERR_ARG, "NULL argument");
  DeviceGuard g(c->device);
  Ctl ctl;
  oes_status st = read_ctl(c, as_stream(stream), &ctl);
  if (st != OES_OK) return st;
  out->steps = ctl.steps;
  out->hits = ctl.hits;
  out->misses = ctl.misses;
  out->evictions = ctl.evictions;
  out->bytes_copied = ctl.bytes;
  out->last_misses = ctl.last_misses;
  out->failed_steps = ctl.failed_steps;
  out->last_indices = ctl.last_indices;
  out->last_missing_full = ctl.last_missing_full;
  out->cpu_experts = ctl.cpu_experts;
  return OES_OK;
}

extern "C" oes_status oes_cache_get_misses(oes_cache *c, int32_t *count, int32_t *slots, int64_t *ids,
                                           int32_t cap, void *stream) {
  if (!c || !count) return fail(OES_ERR_ARG, "NULL argument");
  if (cap < 0) return fail(OES_ERR_ARG, "cap < 0");
  DeviceGuard g(c->device);
  hipStream_t s = as_stream(stream);
  Ctl ctl;
  oes_status st = read_ctl(c, s, &ctl);
  if (st != OES_OK) return st;
  *count = ctl.miss_count;
  int m = std::min(ctl.miss_count, cap);
  if (m > 0 && slots) HIP_TRY(hipMemcpy(slots, c->miss_slot, 4 * (size_t)m, hipMemcpyDeviceToHost));
  if (m > 0 && ids) HIP_TRY(hipMemcpy(ids, c->miss_id, 8 * (size_t)m, hipMemcpyDeviceToHost));
  return OES_OK;
}

extern "C" oes_status oes_cache_fill_slots(oes_cache *c, uint8_t value, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  DeviceGuard g(c->device);
  for (int b = 0; b < c->sc.num_banks; ++b)
    HIP_TRY(hipMemsetAsync(c->slot_bank[b], value, (size_t)c->S * c->sc.bank[b].row_bytes,
                           as_stream(stream)));
  return OES_OK;
}

// ============================================================================ copy
static CopyArgs copy_args(const oes_cache *c, int first_bank, int nbanks) {
  CopyArgs a;
  memset(&a, 0, sizeof(a));
  a.src_table = c->src.d_table;
  a.nb = nbanks;
  a.L = c->sc.num_layers;
  a.E = c->sc.num_experts;
  int prefix = 0;
  for (int i = 0; i < nbanks; ++i) {
    const int b = first_bank + i;
    a.bank[i].slot_base = c->slot_bank[b];
    a.bank[i].row_bytes = c->sc.bank[b].row_bytes;
    a.bank[i].chunks = (int32_t)((c->sc.bank[b].row_bytes + COPY_CHUNK - 1) / COPY_CHUNK);
    a.bank[i].chunk_prefix = prefix;
    a.bank[i].table_col = b;
    prefix += a.bank[i].chunks;
  }
  a.chunks_per_miss = prefix;
  a.err = &c->ctl->err;
  return a;
}

static int copy_grid(const oes_cache *c, int64_t max_items) {
  // 64 blocks of 4 waves keep 2 MiB of host reads in flight, far more than the
  // host link needs; measured, more concurrent streams over the link lower its
  // rate (1024 blocks: 52 GB/s, 64 blocks: 56-57 GB/s on a 57 GB/s link)
  int64_t blocks = c->copy_blocks > 0 ? c->copy_blocks : 64;
  blocks = std::min<int64_t>(blocks, (max_items + 3) / 4);
  return (int)std::max<int64_t>(blocks, 1);
}

static oes_status enqueue_gather(oes_cache *c, const int32_t *count, const int32_t *slots,
                                 const int64_t *ids, const int32_t *gate, int max_entries,
                                 hipStream_t s) {
  if (c->fused_copy) {
    CopyArgs a = copy_args(c, 0, c->sc.num_banks);
    a.count = count; a.slot_list = slots; a.id_list = ids; a.gate = gate;
    HIP_TRY(launch_gather(a, copy_grid(c, (int64_t)max_entries * a.chunks_per_miss), s));
  } else {
    for (int b = 0; b < c->sc.num_banks; ++b) {
      CopyArgs a = copy_args(c, b, 1);
      a.count = count; a.slot_list = slots; a.id_list = ids; a.gate = gate;
      HIP_TRY(launch_gather(a, copy_grid(c, (int64_t)max_entries * a.chunks_per_miss), s));
    }
  }
  return OES_OK;
}

extern "C" oes_status oes_copy_missing(oes_cache *c, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  DeviceGuard g(c->device);
  hipStream_t s = as_stream(stream);
  if (c->copy_mode == OES_COPY_ZERO)
    return enqueue_gather(c, &c->ctl->miss_count, c->miss_slot, c->miss_id, &c->ctl->step_ok, c->maxM, s);
  // DMA mode: the miss list must be known on the host, so this syncs the stream.
  Ctl ctl;
  oes_status st = read_ctl(c, s, &ctl);
  if (st != OES_OK) return st;
  if (!ctl.step_ok || ctl.miss_count == 0) return OES_OK;
  std::vector<int32_t> sl(ctl.miss_count);
  std::vector<int64_t> id(ctl.miss_count);
  HIP_TRY(hipMemcpy(sl.data(), c->miss_slot, 4 * sl.size(), hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(id.data(), c->miss_id, 8 * id.size(), hipMemcpyDeviceToHost));
  const int E = c->sc.num_experts, L = c->sc.num_layers;
  for (int m = 0; m < ctl.miss_count; ++m) {
    const int layer = (int)(id[m] / E), e = (int)(id[m] % E);
    for (int b = 0; b < c->sc.num_banks; ++b) {
      const void *h = c->src.host[(size_t)b * L + layer];
      if (!h) return fail(OES_ERR_ARG, "bank %d has no source for layer %d", b, layer);
      const int64_t rb = c->sc.bank[b].row_bytes;
      HIP_TRY(hipMemcpyAsync(c->slot_bank[b] + (size_t)sl[m] * rb, static_cast<const uint8_t *>(h) + (size_t)e * rb,
                             rb, hipMemcpyHostToDevice, s));
    }
  }
  return OES_OK;
}

extern "C" oes_status oes_cache_load_rows(oes_cache *c, const int32_t *slots, const int64_t *ids,
                                          int32_t count, void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (count < 0 || count > c->S) return fail(OES_ERR_ARG, "count %d outside [0, %d]", count, c->S);
  if (count > 0 && (!slots || !ids)) return fail(OES_ERR_ARG, "NULL list");
  const int64_t nid = (int64_t)c->sc.num_layers * c->sc.num_experts;
  for (int i = 0; i < count; ++i) {
    if (slots[i] < 0 || slots[i] >= c->S) return fail(OES_ERR_ARG, "slot %d out of range", slots[i]);
    if (ids[i] < 0 || ids[i] >= nid) return fail(OES_ERR_ARG, "id %lld out of range", (long long)ids[i]);
    const int layer = (int)(ids[i] / c->sc.num_experts);
    for (int b = 0; b < c->sc.num_banks; ++b)
      if (!c->src.host[(size_t)b * c->sc.num_layers + layer])
        return fail(OES_ERR_ARG, "bank %d has no source for layer %d", b, layer);
  }
  if (count == 0) return OES_OK;
  DeviceGuard g(c->device);
  oes_status st = staging_acquire(c);
  if (st != OES_OK) return st;
  hipStream_t s = as_stream(stream);
  // staging layout for the list: count | slots | ids, after the table area
  uint8_t *p = c->staging + 16 * (size_t)c->S + round_up(sizeof(Ctl), 16);
  int32_t *pc = reinterpret_cast<int32_t *>(p);
  *pc = count;
  memcpy(p + 16, slots, 4 * (size_t)count);
  uint8_t *pid = p + 16 + round_up(4 * (int64_t)count, 16);
  memcpy(pid, ids, 8 * (size_t)count);
  HIP_TRY(hipMemcpyAsync(&c->ctl->aux_count, pc, 4, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->aux_slot, p + 16, 4 * (size_t)count, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->aux_id, pid, 8 * (size_t)count, hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(c->staging_done, s));
  return enqueue_gather(c, &c->ctl->aux_count, c->aux_slot, c->aux_id, nullptr, count, s);
}

// ============================================================================ route
extern "C" oes_status oes_route_workspace(int32_t n, int32_t H, int32_t E, int64_t *bytes) {
  if (!bytes) return fail(OES_ERR_ARG, "bytes is NULL");
  if (n < 0 || H <= 0 || E <= 0) return fail(OES_ERR_ARG, "bad sizes");
  *bytes = round_up(4ll * route_splits(H, E) * n * E + 4ll * n * E, 256);
  return OES_OK;
}

static oes_status check_route(int32_t n, int32_t E, int32_t k, const int32_t *ids, const float *w, bool gemv) {
  if (n < 0) return fail(OES_ERR_ARG, "n < 0");
  if (gemv && (E < 8 || E > 512 || E % 8)) return fail(OES_ERR_ARG, "E must be a multiple of 8 in [8, 512]");
  if (!gemv && (E < 1 || E > 512)) return fail(OES_ERR_ARG, "E must be in [1, 512]");
  if (k < 1 || k > 32 || k > E) return fail(OES_ERR_ARG, "k must be in [1, min(E, 32)]");
  if (n > 0 && (!ids || !w)) return fail(OES_ERR_ARG, "ids / w are NULL");
  return OES_OK;
}

extern "C" oes_status oes_route(const void *x, const void *wg, int32_t n, int32_t H, int32_t E, int32_t k,
                                int32_t *ids, float *w, float *logits, void *workspace,
                                int64_t workspace_bytes, void *stream) {
  oes_status st = check_route(n, E, k, ids, w, true);
  if (st != OES_OK) return st;
  if (H <= 0) return fail(OES_ERR_ARG, "H must be positive");
  if (n == 0) return OES_OK;
  if (!x || !wg || !workspace) return fail(OES_ERR_ARG, "NULL input");
  int64_t need = 0;
  oes_route_workspace(n, H, E, &need);
  if (workspace_bytes < need) return fail(OES_ERR_ARG, "workspace %lld < %lld bytes", (long long)workspace_bytes, (long long)need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(OES_ERR_ARG, "workspace must be 16-byte aligned");
  float *partial = static_cast<float *>(workspace);
  float *lg = logits ? logits : partial + (int64_t)route_splits(H, E) * n * E;
  HIP_TRY(launch_route(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(wg), n, H, E, k, ids,
                       w, lg, partial, as_stream(stream)));
  return OES_OK;
}

extern "C" oes_status oes_route_logits(const float *logits, int32_t n, int32_t E, int32_t k, int32_t *ids,
                                       float *w, void *stream) {
  oes_status st = check_route(n, E, k, ids, w, false);
  if (st != OES_OK) return st;
  if (n == 0) return OES_OK;
  if (!logits) return fail(OES_ERR_ARG, "logits is NULL");
  HIP_TRY(launch_route_logits(logits, n, E, k, ids, w, as_stream(stream)));
  return OES_OK;
}

// ============================================================================ ensure_experts
static oes_status ensure_common(oes_cache *c, int32_t layer, const int32_t *ids, int32_t n, int32_t k,
                                int32_t *slot_ids, int hybrid, int32_t max_fetch, double fetch_fraction,
                                void *stream) {
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (layer < 0 || layer >= c->sc.num_layers) return fail(OES_ERR_ARG, "layer %d outside [0, %d)", layer, c->sc.num_layers);
  if (n < 0 || k < 1) return fail(OES_ERR_ARG, "need n >= 0 and k >= 1");
  if ((int64_t)n * k > 65536) return fail(OES_ERR_ARG, "n*k = %lld exceeds 65536", (long long)n * k);
  if (n > 0 && (!ids || !slot_ids)) return fail(OES_ERR_ARG, "ids / slot_ids are NULL");
  DeviceGuard g(c->device);
  LruArgs a;
  a.owner = c->owner;
  a.stamp = c->stamp;
  a.ctl = c->ctl;
  a.miss_slot = c->miss_slot;
  a.miss_id = c->miss_id;
  a.ids = ids;
  a.slot_ids = slot_ids;
  a.nk = n * k;
  a.layer = layer;
  a.E = c->sc.num_experts;
  a.S = c->S;
  a.Spad = c->Spad;
  a.bpe = c->sc.bytes_per_expert;
  a.hybrid = hybrid;
  a.max_fetch = max_fetch;
  a.fetch_fraction = fetch_fraction;
  HIP_TRY(launch_lru_remap(a, as_stream(stream)));
  return OES_OK;
}

extern "C" oes_status oes_ensure_experts(oes_cache *c, int32_t layer, const int32_t *ids, int32_t n, int32_t k,
                                         int32_t *slot_ids, void *stream) {
  return ensure_common(c, layer, ids, n, k, slot_ids, 0, -1, -1.0, stream);
}

extern "C" oes_status oes_ensure_experts_hybrid(oes_cache *c, int32_t layer, const int32_t *ids, int32_t n,
                                                int32_t k, int32_t *slot_ids, int32_t max_fetch,
                                                double fetch_fraction, void *stream) {
  if (fetch_fraction != fetch_fraction) return fail(OES_ERR_ARG, "fetch_fraction is NaN");
  return ensure_common(c, layer, ids, n, k, slot_ids, 1, max_fetch, fetch_fraction, stream);
}

// ============================================================================ expert FFN
extern "C" oes_status oes_expert_ffn_workspace(const oes_cache *c, int32_t n, int32_t k, int64_t *bytes) {
  if (!c || !bytes) return fail(OES_ERR_ARG, "NULL argument");
  if (n < 0 || k < 1) return fail(OES_ERR_ARG, "need n >= 0 and k >= 1");
  *bytes = expert_ffn_workspace_bytes(n, k, c->sc.hidden, c->sc.inter);
  return OES_OK;
}

// Checks of expert_ffn's arguments other than the workspace; *skip = true for n = 0.
static oes_status ffn_check(const oes_cache *c, const void *x, const int32_t *slot_ids, const float *w, int32_t n,
                            int32_t k, const void *y, bool *skip) {
  *skip = false;
  if (!c) return fail(OES_ERR_ARG, "cache is NULL");
  if (n < 0 || k < 1 || k > 32) return fail(OES_ERR_ARG, "need n >= 0 and 1 <= k <= 32");
  if ((int64_t)n * k > 32768) return fail(OES_ERR_ARG, "n*k exceeds 32768");
  if (n == 0) {
    *skip = true;
    return OES_OK;
  }
  if (!x || !slot_ids || !w || !y) return fail(OES_ERR_ARG, "NULL buffer");
  if (!expert_ffn_supported(c->sc.format, c->sc.hidden, c->sc.inter, k))
    return fail(OES_ERR_UNSUPPORTED, "expert_ffn does not support format %d with H=%d I=%d k=%d", c->sc.format,
                c->sc.hidden, c->sc.inter, k);
  return OES_OK;
}

// Enqueues the FFN kernels with `workspace` (checked by the caller); the cache's device is current.
static oes_status ffn_enqueue(oes_cache *c, const void *x, const int32_t *slot_ids, const float *w, int32_t n,
                              int32_t k, void *y, void *workspace, void *stream) {
  FfnArgs a;
  memset(&a, 0, sizeof(a));
  a.format = c->sc.format;
  a.H = c->sc.hidden;
  a.I = c->sc.inter;
  a.n = n;
  a.k = k;
  a.S = c->S;
  a.E = c->sc.num_experts;
  a.path = c->ffn_path;
  a.x = static_cast<const uint16_t *>(x);
  a.slot_ids = slot_ids;
  a.w = w;
  a.y = static_cast<uint16_t *>(y);
  expert_ffn_carve(a, workspace);
  for (int b = 0; b < c->sc.num_banks; ++b) {
    a.bank[b] = c->slot_bank[b];
    a.row_bytes[b] = c->sc.bank[b].row_bytes;
  }
  a.gate = &c->ctl->step_ok;
  a.err = &c->ctl->err;
  HIP_TRY(launch_expert_ffn(a, as_stream(stream)));
  return OES_OK;
}

extern "C" oes_status oes_expert_ffn(oes_cache *c, const void *x, const int32_t *slot_ids, const float *w,
                                     int32_t n, int32_t k, void *y, void *workspace, int64_t workspace_bytes,
                                     void *stream) {
  bool skip = false;
  oes_status st = ffn_check(c, x, slot_ids, w, n, k, y, &skip);
  if (st != OES_OK || skip) return st;
  if (!workspace) return fail(OES_ERR_ARG, "NULL buffer");
  int64_t need = 0;
  oes_expert_ffn_workspace(c, n, k, &need);
  if (workspace_bytes < need) return fail(OES_ERR_ARG, "workspace %lld < %lld bytes", (long long)workspace_bytes, (long long)need);
  DeviceGuard g(c->device);
  return ffn_enqueue(c, x, slot_ids, w, n, k, y, workspace, stream);
}

extern "C" oes_status oes_expert_ffn_noalloc(oes_cache *c, const void *x, const int32_t *slot_ids, const float *w,
                                             int32_t n, int32_t k, void *y, void *stream) {
  bool skip = false;
  oes_status st = ffn_check(c, x, slot_ids, w, n, k, y, &skip);
  if (st != OES_OK || skip) return st;
  int64_t need = 0;
  oes_expert_ffn_workspace(c, n, k, &need);
  if (need > (int64_t)OES_FFN_NOALLOC_SCRATCH_BYTES)
    return fail(OES_ERR_ARG, "expert_ffn_noalloc: n=%d k=%d needs %lld workspace bytes, more than the %lld-byte "
                "scratch array (use oes_expert_ffn with a workspace)", n, k, (long long)need,
                (long long)OES_FFN_NOALLOC_SCRATCH_BYTES);
  DeviceGuard g(c->device);
  void *ws = nullptr;
  HIP_TRY(ffn_noalloc_scratch(c->device, &ws));
  return ffn_enqueue(c, x, slot_ids, w, n, k, y, ws, stream);
}

// ============================================================================ prefill layers
static void layers_free(oes_layers *p) {
  for (auto b : p->buf)
    if (b) (void)hipFree(b);
  for (auto e : p->ready)
    if (e) (void)hipEventDestroy(e);
  for (auto e : p->released)
    if (e) (void)hipEventDestroy(e);
  p->src.release();
  delete p;
}

extern "C" oes_status oes_layers_create(const oes_schema *sc, int32_t depth, int32_t device, oes_layers **out) {
  if (!out) return fail(OES_ERR_ARG, "out is NULL");
  *out = nullptr;
  oes_status st = check_schema(sc);
  if (st != OES_OK) return st;
  if (depth < 1 || depth > 4) return fail(OES_ERR_ARG, "depth %d outside [1, 4]", depth);
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev) return fail(OES_ERR_ARG, "device %d outside [0, %d)", device, ndev);
  DeviceGuard g(device);
  oes_layers *p = new oes_layers();
  p->sc = *sc;
  p->depth = depth;
  p->device = device;
  p->buf.assign((size_t)depth * sc->num_banks, nullptr);
  p->ready.assign(depth, nullptr);
  p->released.assign(depth, nullptr);
  p->resident.assign(depth, -1);
  for (int d = 0; d < depth; ++d) {
    for (int b = 0; b < sc->num_banks; ++b) {
      e = hipMalloc(&p->buf[(size_t)d * sc->num_banks + b], (size_t)sc->num_experts * sc->bank[b].row_bytes);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        layers_free(p);
        return fail(OES_ERR_NOMEM, "hipMalloc of a layer buffer failed");
      }
    }
    if (hipEventCreateWithFlags(&p->ready[d], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&p->released[d], hipEventDisableTiming) != hipSuccess) {
      layers_free(p);
      return fail(OES_ERR_HIP, "hipEventCreate failed");
    }
  }
  st = p->src.init(sc->num_banks, sc->num_layers);
  if (st != OES_OK) { layers_free(p); return st; }
  *out = p;
  return OES_OK;
}

extern "C" oes_status oes_layers_destroy(oes_layers *p) {
  if (!p) return OES_OK;
  DeviceGuard g(p->device);
  (void)hipDeviceSynchronize();
  layers_free(p);
  return OES_OK;
}

extern "C" oes_status oes_layers_set_source(oes_layers *p, int32_t bank, int32_t layer, const void *host,
                                            int64_t bytes) {
  if (!p) return fail(OES_ERR_ARG, "layers is NULL");
  DeviceGuard g(p->device);
  return p->src.set(p->sc, bank, layer, host, bytes);
}

extern "C" oes_status oes_layers_buffer(const oes_layers *p, int32_t index, int32_t bank, void **dev,
                                        int64_t *bytes) {
  if (!p) return fail(OES_ERR_ARG, "layers is NULL");
  if (index < 0 || index >= p->depth) return fail(OES_ERR_ARG, "buffer index out of range");
  if (bank < 0 || bank >= p->sc.num_banks) return fail(OES_ERR_ARG, "bank out of range");
  if (dev) *dev = p->buf[(size_t)index * p->sc.num_banks + bank];
  if (bytes) *bytes = (int64_t)p->sc.num_experts * p->sc.bank[bank].row_bytes;
  return OES_OK;
}

extern "C" oes_status oes_layers_prefetch(oes_layers *p, int32_t layer, void *copy_stream) {
  if (!p) return fail(OES_ERR_ARG, "layers is NULL");
  if (layer < 0 || layer >= p->sc.num_layers) return fail(OES_ERR_ARG, "layer out of range");
  for (int b = 0; b < p->sc.num_banks; ++b)
    if (!p->src.host[(size_t)b * p->sc.num_layers + layer])
      return fail(OES_ERR_ARG, "bank %d has no source for layer %d", b, layer);
  DeviceGuard g(p->device);
  hipStream_t s = as_stream(copy_stream);
  const int d = layer % p->depth;
  // the previous user of this buffer must have finished
  HIP_TRY(hipStreamWaitEvent(s, p->released[d], 0));
  for (int b = 0; b < p->sc.num_banks; ++b) {
    const int64_t bytes = (int64_t)p->sc.num_experts * p->sc.bank[b].row_bytes;
    HIP_TRY(hipMemcpyAsync(p->buf[(size_t)d * p->sc.num_banks + b], p->src.host[(size_t)b * p->sc.num_layers + layer],
                           bytes, hipMemcpyHostToDevice, s));
  }
  HIP_TRY(hipEventRecord(p->ready[d], s));
  p->resident[d] = layer;
  return OES_OK;
}

extern "C" oes_status oes_layers_ffn_workspace(const oes_layers *p, int32_t n, int32_t k, int64_t *bytes) {
  if (!p || !bytes) return fail(OES_ERR_ARG, "NULL argument");
  if (n < 0 || k < 1) return fail(OES_ERR_ARG, "need n >= 0 and k >= 1");
  *bytes = prefill_workspace_bytes(p->sc.hidden, p->sc.inter, n, k, p->sc.num_experts);
  return OES_OK;
}

extern "C" oes_status oes_layers_ffn(oes_layers *p, int32_t layer, const void *x, const int32_t *ids, const float *w,
                                     int32_t n, int32_t k, void *y, void *workspace, int64_t workspace_bytes,
                                     void *compute_stream) {
  if (!p) return fail(OES_ERR_ARG, "layers is NULL");
  if (p->sc.format != OES_MXFP4_T) return fail(OES_ERR_UNSUPPORTED, "layer FFN is implemented for OES_MXFP4_T");
  if (!prefill_supported(p->sc.hidden, p->sc.inter, p->sc.num_experts))
    return fail(OES_ERR_UNSUPPORTED, "layer FFN needs H and I multiples of 64");
  if (layer < 0 || layer >= p->sc.num_layers) return fail(OES_ERR_ARG, "layer out of range");
  const int d = layer % p->depth;
  if (p->resident[d] != layer) return fail(OES_ERR_STATE, "layer %d was not prefetched", layer);
  if (n < 0 || k < 1 || k > 32) return fail(OES_ERR_ARG, "need n >= 0 and 1 <= k <= 32");
  if ((int64_t)n * k > (1 << 22)) return fail(OES_ERR_ARG, "n*k too large");
  int64_t need = prefill_workspace_bytes(p->sc.hidden, p->sc.inter, n, k, p->sc.num_experts);
  if (n > 0 && (!x || !ids || !w || !y || !workspace)) return fail(OES_ERR_ARG, "NULL buffer");
  if (workspace_bytes < need) return fail(OES_ERR_ARG, "workspace %lld < %lld bytes", (long long)workspace_bytes, (long long)need);
  DeviceGuard g(p->device);
  hipStream_t s = as_stream(compute_stream);
  HIP_TRY(hipStreamWaitEvent(s, p->ready[d], 0));
  if (n > 0) {
    PrefillArgs a;
    memset(&a, 0, sizeof(a));
    a.H = p->sc.hidden;
    a.I = p->sc.inter;
    a.n = n;
    a.k = k;
    a.E = p->sc.num_experts;
    a.x = static_cast<const uint16_t *>(x);
    a.ids = ids;
    a.w = w;
    a.y = static_cast<uint16_t *>(y);
    for (int b = 0; b < p->sc.num_banks; ++b) {
      a.bank[b] = p->buf[(size_t)d * p->sc.num_banks + b];
      a.row_bytes[b] = p->sc.bank[b].row_bytes;
    }
    a.ws = static_cast<uint8_t *>(workspace);
    a.ws_bytes = workspace_bytes;
    HIP_TRY(launch_prefill_ffn(a, s));
  }
  HIP_TRY(hipEventRecord(p->released[d], s));
  return OES_OK;
}

// ============================================================================ probes
static oes_status timed(hipStream_t s, float *ms, hipEvent_t e0, hipEvent_t e1) {
  HIP_TRY(hipEventSynchronize(e1));
  HIP_TRY(hipEventElapsedTime(ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)s;
  return OES_OK;
}

extern "C" oes_status oes_probe_h2d_dma(void *dev, const void *host, int64_t bytes, void *stream, float *ms) {
  if (!dev || !host || bytes <= 0 || !ms) return fail(OES_ERR_ARG, "bad probe arguments");
  hipStream_t s = as_stream(stream);
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  HIP_TRY(hipEventRecord(e0, s));
  HIP_TRY(hipMemcpyAsync(dev, host, bytes, hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(e1, s));
  return timed(s, ms, e0, e1);
}

extern "C" oes_status oes_probe_h2d_kernel(void *dev, const void *host, int64_t bytes, int32_t blocks,
                                           void *stream, float *ms) {
  if (!dev || !host || bytes <= 0 || bytes % 16 || !ms || blocks < 1)
    return fail(OES_ERR_ARG, "bad probe arguments");
  const void *d = device_view_of_host(host);
  if (!d) return fail(OES_ERR_ARG, "host buffer is not pinned");
  hipStream_t s = as_stream(stream);
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  HIP_TRY(hipEventRecord(e0, s));
  HIP_TRY(launch_stream_copy(static_cast<uint8_t *>(dev), static_cast<const uint8_t *>(d), bytes, blocks, s));
  HIP_TRY(hipEventRecord(e1, s));
  return timed(s, ms, e0, e1);
}

extern "C" oes_status oes_probe_hbm_read(const void *dev, int64_t bytes, int64_t stride, int32_t count, void *sink,
                                         void *stream, float *ms) {
  if (!dev || bytes <= 0 || bytes % 16 || stride < 0 || stride % 16 || count < 1 || !sink || !ms)
    return fail(OES_ERR_ARG, "bad probe arguments");
  hipStream_t s = as_stream(stream);
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  HIP_TRY(hipEventRecord(e0, s));
  for (int32_t i = 0; i < count; ++i)
    HIP_TRY(launch_hbm_read(static_cast<const uint8_t *>(dev) + (int64_t)i * stride, bytes, static_cast<float *>(sink), s));
  HIP_TRY(hipEventRecord(e1, s));
  const oes_status st = timed(s, ms, e0, e1);
  if (st == OES_OK) *ms /= (float)count;
  return st;
}

static oes_status probe_mfma(bool f8f4, int32_t blocks, int32_t iters, void *sink, void *stream, float *ms,
                             double *flops) {
  if (blocks < 1 || iters < 1 || iters > (1 << 24) || !sink || !ms || !flops)
    return fail(OES_ERR_ARG, "bad probe arguments");
  hipStream_t s = as_stream(stream);
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  HIP_TRY(hipEventRecord(e0, s));
  HIP_TRY(launch_mfma_probe(f8f4, blocks, iters, static_cast<float *>(sink), s));
  HIP_TRY(hipEventRecord(e1, s));
  *flops = (double)mfma_probe_flops(f8f4, blocks, iters);
  return timed(s, ms, e0, e1);
}

extern "C" oes_status oes_probe_mfma_bf16(int32_t blocks, int32_t iters, void *sink, void *stream, float *ms,
                                          double *flops) {
  return probe_mfma(false, blocks, iters, sink, stream, ms, flops);
}

extern "C" oes_status oes_probe_mfma_f8f4(int32_t blocks, int32_t iters, void *sink, void *stream, float *ms,
                                          double *flops) {
  return probe_mfma(true, blocks, iters, sink, stream, ms, flops);
}

// ============================================================================ hybrid step
namespace oes {
const oes_schema *cpu_moe_schema(const oes_cpu_moe *m);  // cpu_moe.cpp
}

// Host workspace of a hybrid step: x bf16 [n, H] | ids | slot_ids | w [n, k] | y_cpu fp32 [n, H].
struct HybridHost {
  int64_t x, ids, slots, w, y, total;
};
static HybridHost hybrid_host_layout(int64_t n, int64_t k, int64_t H) {
  HybridHost l;
  int64_t off = 0;
  l.x = off;     off = round_up(off + 2 * n * H, 64);
  l.ids = off;   off = round_up(off + 4 * n * k, 64);
  l.slots = off; off = round_up(off + 4 * n * k, 64);
  l.w = off;     off = round_up(off + 4 * n * k, 64);
  l.y = off;     off = round_up(off + 4 * n * H, 64);
  l.total = off;
  return l;
}

extern "C" oes_status oes_hybrid_workspace(const oes_cache *c, int32_t n, int32_t k, int64_t *host_bytes,
                                           int64_t *dev_bytes) {
  if (!c || !host_bytes || !dev_bytes) return fail(OES_ERR_ARG, "NULL argument");
  if (n < 0 || k < 1) return fail(OES_ERR_ARG, "need n >= 0 and k >= 1");
  *host_bytes = hybrid_host_layout(n, k, c->sc.hidden).total;
  *dev_bytes = round_up(4ll * n * c->sc.hidden, 64);
  return OES_OK;
}

extern "C" oes_status oes_hybrid_step(oes_cache *c, oes_cpu_moe *cpu, int32_t layer, const void *x,
                                      const int32_t *ids, const float *w, int32_t n, int32_t k, int32_t *slot_ids,
                                      void *y, void *ffn_ws, int64_t ffn_ws_bytes, void *host_ws,
                                      int64_t host_ws_bytes, void *dev_ws, int64_t dev_ws_bytes,
                                      int32_t max_fetch, double fetch_fraction, void *stream) {
  if (!c || !cpu) return fail(OES_ERR_ARG, "cache or executor is NULL");
  if (memcmp(oes::cpu_moe_schema(cpu), &c->sc, sizeof(oes_schema)) != 0)
    return fail(OES_ERR_ARG, "the executor and the cache have different schemas");
  if (n < 0 || k < 1 || k > 32) return fail(OES_ERR_ARG, "need n >= 0 and 1 <= k <= 32");
  if (n == 0) return OES_OK;
  if (!x || !ids || !w || !slot_ids || !y || !host_ws || !dev_ws) return fail(OES_ERR_ARG, "NULL buffer");
  const int H = c->sc.hidden;
  const HybridHost l = hybrid_host_layout(n, k, H);
  if (host_ws_bytes < l.total) return fail(OES_ERR_ARG, "host workspace %lld < %lld bytes", (long long)host_ws_bytes, (long long)l.total);
  if (dev_ws_bytes < 4ll * n * H) return fail(OES_ERR_ARG, "device workspace %lld < %lld bytes", (long long)dev_ws_bytes, 4ll * n * H);
  DeviceGuard g(c->device);
  if (!g.ok) return fail(OES_ERR_HIP, "hipSetDevice(%d) failed", c->device);
  hipStream_t s = as_stream(stream);
  if (!c->hybrid_ev) HIP_TRY(hipEventCreateWithFlags(&c->hybrid_ev, hipEventDisableTiming));
  uint8_t *hw = static_cast<uint8_t *>(host_ws);
  // 1. the remap, and the step's routing on its way to the host
  oes_status st = oes_ensure_experts_hybrid(c, layer, ids, n, k, slot_ids, max_fetch, fetch_fraction, stream);
  if (st != OES_OK) return st;
  HIP_TRY(hipMemcpyAsync(hw + l.x, x, 2 * (size_t)n * H, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(hw + l.ids, ids, 4 * (size_t)n * k, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(hw + l.slots, slot_ids, 4 * (size_t)n * k, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(hw + l.w, w, 4 * (size_t)n * k, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipEventRecord(c->hybrid_ev, s));
  // 2. the GPU part: fetch the capped misses, FFN over the slot pairs (-1 pairs skipped)
  st = oes_copy_missing(c, stream);
  if (st != OES_OK) return st;
  st = oes_expert_ffn(c, x, slot_ids, w, n, k, y, ffn_ws, ffn_ws_bytes, stream);
  if (st != OES_OK) return st;
  // 3. the CPU part, while the GPU copies
  HIP_TRY(hipEventSynchronize(c->hybrid_ev));
  const int32_t *hs = reinterpret_cast<const int32_t *>(hw + l.slots);
  bool any = false;
  for (int64_t i = 0; i < (int64_t)n * k; ++i) any = any || hs[i] < 0;
  if (!any) return OES_OK;
  float *yc = reinterpret_cast<float *>(hw + l.y);
  st = oes_cpu_moe_run(cpu, layer, hw + l.x, reinterpret_cast<const int32_t *>(hw + l.ids), hs,
                       reinterpret_cast<const float *>(hw + l.w), n, k, yc);
  if (st != OES_OK) return st;
  // 4. y += y_cpu, after the GPU FFN in stream order
  HIP_TRY(hipMemcpyAsync(dev_ws, yc, 4 * (size_t)n * H, hipMemcpyHostToDevice, s));
  HIP_TRY(launch_add_to_bf16(static_cast<uint16_t *>(y), static_cast<const float *>(dev_ws), (int64_t)n * H, s));
  return OES_OK;
}

extern "C" oes_status oes_combine_cpu(void *y_bf16, const float *y_cpu, int64_t count, void *stream) {
  if (count < 0) return fail(OES_ERR_ARG, "count < 0");
  if (count == 0) return OES_OK;
  if (!y_bf16 || !y_cpu) return fail(OES_ERR_ARG, "NULL buffer");
  HIP_TRY(launch_add_to_bf16(static_cast<uint16_t *>(y_bf16), y_cpu, count, as_stream(stream)));
  return OES_OK;
}

extern "C" oes_status oes_debug_decode(int32_t elem, const void *codes, int32_t n, float *out, void *stream) {
  if (n < 0) return fail(OES_ERR_ARG, "n < 0");
  if (n == 0) return OES_OK;
  if (!codes || !out) return fail(OES_ERR_ARG, "NULL buffer");
  if (elem != OES_ELEM_E4M3 && elem != OES_ELEM_FP4X2 && elem != OES_ELEM_E8M0 && elem != OES_ELEM_BF16 &&
      elem != OES_ELEM_FP16 && elem != OES_ELEM_Q4X2)
    return fail(OES_ERR_ARG, "unsupported element type %d", elem);
  if (elem == OES_ELEM_Q4X2 && n % 32)
    return fail(OES_ERR_ARG, "q4x2 codes come in blocks of 32 elements (n = %d)", n);
  HIP_TRY(launch_debug_decode(elem, static_cast<const uint8_t *>(codes), n, out, as_stream(stream)));
  return OES_OK;
}
