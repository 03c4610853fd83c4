// Internal definitions shared by the host API and the HIP kernels of liboes.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/oes.h"

namespace oes {

// Leaves msg in the thread-local error string read by oes_last_error (host_common.cpp).
oes_status set_error(oes_status st, const char *msg);

// Device-side control block of one slot cache (one per cache, in HBM).
struct Ctl {
  uint64_t clock;        // LRU clock: stamp given to the slots of the last step
  int32_t err;           // sticky device error (OES_ERR_*), cleared by oes_cache_check
  int32_t step_ok;       // 0 after a failed ensure_experts (copy and FFN skip); 1 otherwise
  int32_t miss_count;    // entries in the miss list of the last step
  int32_t aux_count;     // entries in the host-driven load list
  uint64_t steps, hits, misses, evictions, bytes;
  uint32_t last_misses;
  int32_t failed_steps;
  uint32_t last_indices;       // hybrid: misses fetched by the last step (within the cap)
  uint32_t last_missing_full;  // hybrid: misses of the last step before the cap
  uint64_t cpu_experts;        // hybrid: misses left to the CPU executor, summed over steps
};

// ---------------------------------------------------------------- ensure_experts
struct LruArgs {
  int64_t *owner;
  uint64_t *stamp;
  Ctl *ctl;
  int32_t *miss_slot;
  int64_t *miss_id;
  const int32_t *ids;
  int32_t *slot_ids;
  int32_t nk, layer, E, S, Spad;
  int64_t bpe;
  int32_t hybrid;          // 1: ensure_experts_hybrid (fetch cap; overflow requests map to -1)
  int32_t max_fetch;       // hybrid cap if >= 0
  double fetch_fraction;   // else the share of the misses to fetch if >= 0, else a cap of one
};
hipError_t launch_lru_remap(const LruArgs &a, hipStream_t s);
// step_ok = 1, miss_count = 0 (a one-thread kernel, safe under graph capture)
void launch_reset_step(Ctl *ctl, hipStream_t s);

// ---------------------------------------------------------------- copy (gather)
struct CopyBank {
  uint8_t *slot_base;   // device slot bank
  int64_t row_bytes;    // bytes per expert row
  int32_t chunks;       // chunks of this bank per miss
  int32_t chunk_prefix; // chunks of the banks before this one
  int32_t table_col;    // column of this bank in the source table
  int32_t pad;
};
struct CopyArgs {
  const uint64_t *src_table;  // [banks_total][L] device-readable host addresses, 0 = none
  CopyBank bank[OES_MAX_BANKS];
  int32_t nb, L, E, chunks_per_miss;
  const int32_t *count;       // device: number of list entries
  const int32_t *slot_list;   // device
  const int64_t *id_list;     // device
  const int32_t *gate;        // device step_ok flag, or nullptr (always run)
  int32_t *err;               // device sticky error
};
constexpr int COPY_UNROLL = 8;                       // 16-byte loads in flight per lane
constexpr int64_t COPY_CHUNK = 64 * 16 * COPY_UNROLL;  // bytes one wave moves per work item
hipError_t launch_gather(const CopyArgs &a, int blocks, hipStream_t s);
// new_bank row i <- old_bank row src[i] for i < n (src[i] = -1: skipped); src on the device
hipError_t launch_slot_move(uint8_t *dst, const uint8_t *src_bank, const int32_t *src, int n, int64_t row_bytes,
                            hipStream_t s);

// ---------------------------------------------------------------- route
int route_splits(int H, int E);
hipError_t launch_route(const uint16_t *x, const uint16_t *wg, int n, int H, int E, int k,
                        int32_t *ids, float *w, float *logits, float *partial, hipStream_t s);
hipError_t launch_route_logits(const float *logits, int n, int E, int k, int32_t *ids, float *w,
                               hipStream_t s);

// ---------------------------------------------------------------- decode FFN
struct FfnArgs {
  int32_t format;
  int32_t H, I, n, k, S;
  int32_t E;                             // experts per layer (chooses the grouped path)
  int32_t path;                          // OES_FFN_AUTO / OES_FFN_PER_PAIR / OES_FFN_GROUPED
  const uint16_t *x;
  const int32_t *slot_ids;
  const float *w;
  uint16_t *y;
  uint16_t *h;                           // workspace: bf16 h rows [n*k, I]
  float *o;                              // n >= 2: each pair's down output [n*k, H] (fp32)
  int32_t *grp;                          // n >= 2: pairs grouped by slot (count, slots, starts, pairs)
  const uint8_t *bank[OES_MAX_BANKS];    // slot banks
  int64_t row_bytes[OES_MAX_BANKS];
  const int32_t *gate;                   // step_ok, or nullptr
  int32_t *err;
};
// Workspace bytes of the decode FFN for n tokens with top-k, and its carving into h / o / grp.
int64_t expert_ffn_workspace_bytes(int n, int k, int H, int I);
void expert_ffn_carve(FfnArgs &a, void *workspace);
// Returns hipErrorInvalidValue when the shape cannot be tiled (caller maps it to UNSUPPORTED).
hipError_t launch_expert_ffn(const FfnArgs &a, hipStream_t s);
// Device address of the file-scope FFN scratch array on the current device
// (looked up once per device; nullptr and the HIP error on failure).
hipError_t ffn_noalloc_scratch(int device, void **ptr);
bool expert_ffn_supported(int format, int H, int I, int k);

// ---------------------------------------------------------------- prefill grouped FFN (MXFP4)
struct PrefillArgs {
  int32_t H, I, n, k, E;
  const uint16_t *x;          // [n, H] bf16
  const int32_t *ids;         // [n, k]
  const float *w;             // [n, k]
  uint16_t *y;                // [n, H] bf16
  const uint8_t *bank[OES_MAX_BANKS];  // layer buffer: row e = expert e
  int64_t row_bytes[OES_MAX_BANKS];
  uint8_t *ws;                // workspace
  int64_t ws_bytes;
};
bool prefill_supported(int H, int I, int E);
int64_t prefill_workspace_bytes(int H, int I, int n, int k, int E);
hipError_t launch_prefill_ffn(const PrefillArgs &a, hipStream_t s);

// ---------------------------------------------------------------- probes
hipError_t launch_stream_copy(uint8_t *dst, const uint8_t *src, int64_t bytes, int blocks,
                              hipStream_t s);
hipError_t launch_hbm_read(const uint8_t *src, int64_t bytes, float *sink, hipStream_t s);
// f8f4: the block-scaled e4m3 x e2m1 MFMA of the prefill GEMM; else the bf16 MFMA
hipError_t launch_mfma_probe(bool f8f4, int blocks, int iters, float *sink, hipStream_t s);
int64_t mfma_probe_flops(bool f8f4, int blocks, int iters);

// ---------------------------------------------------------------- debug decode
// y[i] = bf16_rne(float(y[i]) + add[i]) for i < count (device buffers)
hipError_t launch_add_to_bf16(uint16_t *y, const float *add, int64_t count, hipStream_t s);
// out[i] = value of element i of `elem` codes (fp4x2: 2 per byte, element 2j low nibble)
hipError_t launch_debug_decode(int elem, const uint8_t *codes, int n, float *out, hipStream_t s);

}  // namespace oes
