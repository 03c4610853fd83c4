// Host-only basics of liboes.so: the thread-local error message, status names,
// the ABI version and the bank schemas (bank_specs).  Plain C++ (no HIP), so the
// host-only parts of the library can also be built on their own, e.g. with the
// address and undefined-behaviour sanitizers.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/oes.h"

namespace oes {
oes_status set_error(oes_status st, const char *msg);
}

namespace {

thread_local std::string g_err;

oes_status fail(oes_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
oes_status fail(oes_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

void set_spec(oes_bank_spec *b, const char *name, int elem, int ndim, int64_t d0, int64_t d1,
              int64_t d2, int64_t row_bytes) {
  memset(b, 0, sizeof(*b));
  snprintf(b->name, sizeof(b->name), "%s", name);
  b->elem = elem;
  b->ndim = ndim;
  b->shape[0] = d0;
  b->shape[1] = d1;
  b->shape[2] = d2;
  b->row_bytes = row_bytes;
}

}  // namespace

namespace oes {
// Leaves msg in the thread-local error string read by oes_last_error.
oes_status set_error(oes_status st, const char *msg) {
  g_err = msg;
  return st;
}
}  // namespace oes

// ============================================================================ basics
extern "C" const char *oes_status_str(oes_status s) {
  switch (s) {
    case OES_OK: return "OES_OK";
    case OES_ERR_ARG: return "OES_ERR_ARG";
    case OES_ERR_CAPACITY: return "OES_ERR_CAPACITY";
    case OES_ERR_HIP: return "OES_ERR_HIP";
    case OES_ERR_NOMEM: return "OES_ERR_NOMEM";
    case OES_ERR_STATE: return "OES_ERR_STATE";
    case OES_ERR_UNSUPPORTED: return "OES_ERR_UNSUPPORTED";
    default: return "OES_ERR_UNKNOWN";
  }
}

extern "C" const char *oes_last_error(void) { return g_err.c_str(); }
extern "C" int32_t oes_abi_version(void) { return OES_ABI_VERSION; }

// ============================================================================ schema
extern "C" oes_status oes_schema_make(int32_t format, int32_t L, int32_t E, int32_t H, int32_t I,
                                      oes_schema *out) {
  if (!out) return fail(OES_ERR_ARG, "out is NULL");
  if (L <= 0 || E <= 0 || H <= 0 || I <= 0)
    return fail(OES_ERR_ARG, "L, E, H, I must be positive (got %d, %d, %d, %d)", L, E, H, I);
  if (E > OES_MAX_EXPERTS) return fail(OES_ERR_ARG, "E = %d exceeds %d", E, OES_MAX_EXPERTS);
  if ((int64_t)L * E >= (1ll << 40)) return fail(OES_ERR_ARG, "L*E too large");
  oes_schema sc;
  memset(&sc, 0, sizeof(sc));
  sc.format = format;
  sc.num_layers = L;
  sc.num_experts = E;
  sc.hidden = H;
  sc.inter = I;
  const int64_t h = H, i2 = 2ll * I, i = I;
  switch (format) {
    case OES_BF16:
      if (H % 8 || I % 8) return fail(OES_ERR_ARG, "bf16 needs H and I multiples of 8");
      sc.num_banks = 2;
      set_spec(&sc.bank[0], "gate_up", OES_ELEM_BF16, 2, i2, h, 0, i2 * h * 2);
      set_spec(&sc.bank[1], "down", OES_ELEM_BF16, 2, h, i, 0, h * i * 2);
      break;
    case OES_FP8_BLOCK128:
      if (H % 128 || I % 128) return fail(OES_ERR_ARG, "fp8 block needs H and I multiples of 128");
      sc.num_banks = 4;
      set_spec(&sc.bank[0], "gate_up", OES_ELEM_E4M3, 2, i2, h, 0, i2 * h);
      set_spec(&sc.bank[1], "gate_up_scale", OES_ELEM_F32, 2, i2 / 128, h / 128, 0, (i2 / 128) * (h / 128) * 4);
      set_spec(&sc.bank[2], "down", OES_ELEM_E4M3, 2, h, i, 0, h * i);
      set_spec(&sc.bank[3], "down_scale", OES_ELEM_F32, 2, h / 128, i / 128, 0, (h / 128) * (i / 128) * 4);
      break;
    case OES_NVFP4:
      if (H % 32 || I % 32) return fail(OES_ERR_ARG, "nvfp4 needs H and I multiples of 32");
      sc.num_banks = 6;
      set_spec(&sc.bank[0], "gate_up_codes", OES_ELEM_FP4X2, 2, i2, h / 2, 0, i2 * h / 2);
      set_spec(&sc.bank[1], "gate_up_scale", OES_ELEM_E4M3, 2, i2, h / 16, 0, i2 * h / 16);
      set_spec(&sc.bank[2], "gate_up_global", OES_ELEM_FP16, 1, i2, 0, 0, i2 * 2);
      set_spec(&sc.bank[3], "down_codes", OES_ELEM_FP4X2, 2, h, i / 2, 0, h * i / 2);
      set_spec(&sc.bank[4], "down_scale", OES_ELEM_E4M3, 2, h, i / 16, 0, h * i / 16);
      set_spec(&sc.bank[5], "down_global", OES_ELEM_FP16, 1, h, 0, 0, h * 2);
      break;
    case OES_MXFP4_T:
      if (H % 32 || I % 32) return fail(OES_ERR_ARG, "mxfp4 needs H and I multiples of 32");
      sc.num_banks = 6;
      set_spec(&sc.bank[0], "gate_up_blocks", OES_ELEM_U8, 3, h / 32, i2, 16, (h / 32) * i2 * 16);
      set_spec(&sc.bank[1], "gate_up_scales", OES_ELEM_E8M0, 2, h / 32, i2, 0, (h / 32) * i2);
      set_spec(&sc.bank[2], "gate_up_bias", OES_ELEM_BF16, 1, i2, 0, 0, i2 * 2);
      set_spec(&sc.bank[3], "down_blocks", OES_ELEM_U8, 3, i / 32, h, 16, (i / 32) * h * 16);
      set_spec(&sc.bank[4], "down_scales", OES_ELEM_E8M0, 2, i / 32, h, 0, (i / 32) * h);
      set_spec(&sc.bank[5], "down_bias", OES_ELEM_BF16, 1, h, 0, 0, h * 2);
      break;
    case OES_Q4_0:
      if (H % 32 || I % 32) return fail(OES_ERR_ARG, "q4_0 needs H and I multiples of 32");
      sc.num_banks = 4;
      set_spec(&sc.bank[0], "gate_up_q", OES_ELEM_Q4X2, 2, i2, h / 2, 0, i2 * h / 2);
      set_spec(&sc.bank[1], "gate_up_d", OES_ELEM_FP16, 2, i2, h / 32, 0, i2 * (h / 32) * 2);
      set_spec(&sc.bank[2], "down_q", OES_ELEM_Q4X2, 2, h, i / 2, 0, h * i / 2);
      set_spec(&sc.bank[3], "down_d", OES_ELEM_FP16, 2, h, i / 32, 0, h * (i / 32) * 2);
      break;
    default:
      return fail(OES_ERR_ARG, "unknown format %d", format);
  }
  for (int b = 0; b < sc.num_banks; ++b) {
    if (sc.bank[b].row_bytes % 16)
      return fail(OES_ERR_ARG, "bank %s: row of %lld bytes is not a multiple of 16", sc.bank[b].name,
                  (long long)sc.bank[b].row_bytes);
    sc.bytes_per_expert += sc.bank[b].row_bytes;
  }
  *out = sc;
  return OES_OK;
}

