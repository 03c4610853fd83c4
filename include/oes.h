/*
 * oes.h - C ABI of liboes.so: offloaded expert slots on an MI355X (gfx950).
 *
 * The per-layer MoE expert step of an offloaded-expert inference engine:
 *
 *   route -> ensure_experts -> copy_missing -> expert_ffn
 *
 * Expert weights live in caller-owned pinned host memory as "banks", one bank
 * per schema tensor, each bank supplied as one host tensor per layer; the GPU
 * keeps one slot cache shared by every layer; each step remaps the routed
 * experts (flat id = layer * E + expert) onto slots with a global LRU, gathers
 * the missing experts' rows from every bank in one fused copy, and runs the
 * SwiGLU expert FFN on the slot cache.  (FreeToken architecture walk-through
 * §5; FreeToken MoE benchmark guide §1 background, §4.1-§4.4.)  Prefill
 * streams whole layers through a two-deep device buffer so copy and compute
 * overlap (architecture walk-through §5).
 *
 * Conventions for every function:
 *   - returns oes_status: OES_OK (0) or a negative error; never throws, never
 *     aborts; on error oes_last_error() holds a thread-local message;
 *   - argument errors are detected before any GPU work and change no state;
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream);
 *     step calls only enqueue work on it and never synchronise; calls that
 *     return device-side results to the host say "syncs" and synchronise it;
 *   - device pointers are plain device addresses (e.g. torch tensor data);
 *     host pointers are plain host addresses;
 *   - a cache is not thread-safe: use it from one thread and one stream.
 *
 * Weights use the [out, in] convention: gate_up is [2I, H] (rows [0, I) gate,
 * rows [I, 2I) up) and down is [H, I]; activations are bf16 [n, H] row-major.
 */
#ifndef OES_H_
#define OES_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OES_ABI_VERSION 1

typedef int32_t oes_status;
enum {
  OES_OK = 0,
  OES_ERR_ARG = -1,         /* bad argument; nothing done */
  OES_ERR_CAPACITY = -2,    /* more distinct experts in a step than slots */
  OES_ERR_HIP = -3,         /* a HIP runtime call failed (message has hipGetErrorString) */
  OES_ERR_NOMEM = -4,       /* device or host allocation failed */
  OES_ERR_STATE = -5,       /* call not valid in the object's current state */
  OES_ERR_UNSUPPORTED = -6  /* format / size combination not implemented */
};

/* Static string for a status code. */
const char *oes_status_str(oes_status s);
/* Thread-local detail message of the last failing call on this thread ("" if none). */
const char *oes_last_error(void);
/* OES_ABI_VERSION of the loaded library. */
int32_t oes_abi_version(void);

/* ------------------------------------------------------------------ schema */
/*
 * Bank schema (FreeToken MoE benchmark guide §4.2; architecture walk-through
 * §5): every format declares its own list of banks, one row per expert per
 * bank; the cache moves rows and does not care about their layout.
 *
 *   OES_BF16          gate_up [2I,H] bf16, down [H,I] bf16
 *   OES_FP8_BLOCK128  gate_up [2I,H] e4m3, gate_up_scale [2I/128,H/128] f32,
 *                     down [H,I] e4m3, down_scale [H/128,I/128] f32
 *                     (W = e4m3(q) * scale of its 128x128 block)
 *   OES_NVFP4         gate_up_codes [2I,H/2] (two e2m1 per byte, element 2j in
 *                     the low nibble), gate_up_scale [2I,H/16] e4m3,
 *                     gate_up_global [2I] fp16, then the same three for down
 *                     (W = e2m1 * e4m3 scale of its 16-block * fp16 row global)
 *   OES_MXFP4_T       gate_up_blocks [H/32,2I,16] u8 (32 e2m1 codes along K per
 *                     16 bytes), gate_up_scales [H/32,2I] e8m0, gate_up_bias
 *                     [2I] bf16, then the same three for down over [I/32,H,16]
 *                     (W[n,c] = e2m1 * 2^(scale-127); bias added after the matmul)
 *   OES_Q4_0          gate_up_q [2I,H/2] (GGUF block_q4_0 codes: in every 16
 *                     bytes, byte j holds element j in its low nibble and
 *                     element j+16 in its high nibble), gate_up_d [2I,H/32] fp16,
 *                     down_q [H,I/2], down_d [H,I/32] (W = (q - 8) * d of its
 *                     32-block; the fifth format of FreeToken architecture
 *                     walk-through §5, GGUF Q4_0 MoE in §6)
 */
enum { OES_BF16 = 0, OES_FP8_BLOCK128 = 1, OES_NVFP4 = 2, OES_MXFP4_T = 3, OES_Q4_0 = 4 };
enum {
  OES_ELEM_BF16 = 0, OES_ELEM_E4M3 = 1, OES_ELEM_F32 = 2, OES_ELEM_FP4X2 = 3,
  OES_ELEM_FP16 = 4, OES_ELEM_E8M0 = 5, OES_ELEM_U8 = 6, OES_ELEM_Q4X2 = 7
};
#define OES_MAX_BANKS 6
#define OES_MAX_SLOTS 4096     /* slot pool limit of the single-workgroup remap */
#define OES_MAX_EXPERTS 4096   /* experts per layer */

typedef struct {
  char name[24];        /* e.g. "gate_up_codes" */
  int32_t elem;         /* OES_ELEM_* */
  int32_t ndim;         /* 1..3 */
  int64_t shape[3];     /* row shape; for FP4X2 the last dim counts bytes */
  int64_t row_bytes;    /* bytes of one expert's row (always a multiple of 16) */
} oes_bank_spec;

typedef struct {
  int32_t format, num_layers, num_experts, hidden, inter, num_banks;
  oes_bank_spec bank[OES_MAX_BANKS];
  int64_t bytes_per_expert;  /* sum of row_bytes over the banks */
} oes_schema;

/* Fill *out with the bank list of a format (the pages' bank_specs()).
 * Errors: OES_ERR_ARG for L, E, H, I <= 0, E > OES_MAX_EXPERTS, sizes the
 * format cannot tile (bf16: H, I multiples of 8; fp8: of 128; nvfp4, mxfp4
 * and q4_0: of 32), or an unknown format.  Pure host code, no GPU needed. */
oes_status oes_schema_make(int32_t format, int32_t num_layers, int32_t num_experts,
                           int32_t hidden, int32_t inter, oes_schema *out);

/* ------------------------------------------------------------------ slot cache */
typedef struct oes_cache oes_cache;

typedef struct {
  uint64_t steps;         /* successful ensure_experts calls */
  uint64_t hits;          /* distinct requested ids already resident */
  uint64_t misses;        /* distinct requested ids installed */
  uint64_t evictions;     /* misses that displaced a non-empty slot */
  uint64_t bytes_copied;  /* misses * bytes_per_expert */
  uint32_t last_misses;   /* misses of the last successful step (installed ones) */
  int32_t failed_steps;   /* ensure_experts calls that failed on the device */
  uint32_t last_indices;       /* misses fetched by the last step (num_indices) */
  uint32_t last_missing_full;  /* misses of the last step before a hybrid cap (num_missing_full) */
  uint64_t cpu_experts;        /* hybrid: misses left to the CPU executor, summed */
} oes_stats;

/* Create a slot cache of num_slots experts on HIP device `device`
 * (architecture walk-through §5; benchmark guide §1: one unified slot cache).
 * The cache owns: one HBM slot bank per schema bank (num_slots rows each), the
 * slot table (owner int64 = flat id or -1, stamp uint64, a clock), the miss
 * list and a device status word.  Initial state: every slot empty, stamps 0,
 * clock 0; slot bytes are undefined until written.
 * Errors: OES_ERR_ARG (null, num_slots < 1 or > OES_MAX_SLOTS, bad schema),
 * OES_ERR_NOMEM, OES_ERR_HIP. */
oes_status oes_cache_create(const oes_schema *schema, int32_t num_slots, int32_t device,
                            oes_cache **out);
/* Free everything the cache owns (after synchronising its device).  NULL is OK. */
oes_status oes_cache_destroy(oes_cache *c);

/* Register the host tensor holding bank `bank` of layer `layer`: E rows of
 * row_bytes each, contiguous, expert-major (benchmark guide §4.4: each bank's
 * sources are a per-layer list).  `host` must be pinned host memory the
 * device can read (hipHostMalloc / torch pin_memory), 16-byte aligned, and
 * must outlive the cache; it stays caller-owned.  bytes must equal
 * E * row_bytes.  Errors: OES_ERR_ARG (range, size, alignment, memory that is
 * not pinned host memory), OES_ERR_HIP. */
oes_status oes_cache_set_source(oes_cache *c, int32_t bank, int32_t layer, const void *host,
                                int64_t bytes);

/* Overwrite the slot table (the benchmark's prepare_state, benchmark guide
 * §4.3) from host arrays of num_slots entries; clears the device status and
 * miss list.  owner[s] must be -1 or in [0, 2^50); stamp[s] < 2^62 and
 * clock < 2^62.  Enqueued on `stream` (host arrays are copied before return). */
oes_status oes_cache_set_state(oes_cache *c, const int64_t *owner, const uint64_t *stamp,
                               uint64_t clock, void *stream);
/* Device-side snapshot of the slot table (owners, stamps, clock): snapshot
 * copies the live table into a cache-owned device buffer, restore copies it
 * back and clears the miss list and the step status (the sticky error is
 * kept).  Device-to-device copies enqueued on `stream`, no host sync: lets a
 * caller re-run a step from the same state many times back to back (the copy
 * benchmark's repeats, benchmark guide §4.3).  restore before any snapshot
 * returns OES_ERR_STATE. */
oes_status oes_cache_snapshot(oes_cache *c, void *stream);
oes_status oes_cache_restore(oes_cache *c, void *stream);

/* Resize the slot pool to num_slots slots at run time, keeping the resident
 * experts' bytes (no reload from the host banks) and their LRU order
 * (FreeToken architecture walk-through §4: VRAM moves between the expert cache
 * and other uses with no restart and no weight reload).
 *   grow:   every slot keeps its index, contents, owner and stamp; the new
 *           slots are empty (their bytes are undefined until a copy fills them).
 *   shrink: the kept slots are the num_slots that come last in the remap's
 *           victim order (empty slots leave first, then the least recently
 *           used: key (not empty, stamp, owner, slot)); they move, in
 *           ascending old index, to slots [0, num_slots).  The experts of the
 *           other slots are no longer resident.
 * Stamps, clock and the counters of oes_cache_stats are kept; the miss list of
 * the last step and the load list are cleared (copy_missing then moves
 * nothing), and a snapshot is discarded (restore returns OES_ERR_STATE).  A
 * resize to the current size changes nothing.
 * slot_ids of earlier steps name old slots: remap before the next FFN.
 * Synchronous: syncs `stream` first (every enqueued step finishes), moves the
 * rows with a device kernel, syncs again.  New banks and table are allocated
 * before the old ones are freed, so the device briefly holds both; on any
 * error the cache is unchanged.  Errors: OES_ERR_ARG (num_slots outside
 * [1, OES_MAX_SLOTS]), OES_ERR_NOMEM, OES_ERR_HIP. */
oes_status oes_cache_resize(oes_cache *c, int32_t num_slots, void *stream);

/* Read the slot table into host arrays of num_slots entries (any pointer may
 * be NULL): the state the benchmark prepares and the LRU maintains (benchmark
 * guide §4.3; architecture walk-through §5: the unified slot cache).  Syncs
 * `stream`. */
oes_status oes_cache_get_state(oes_cache *c, int64_t *owner, uint64_t *stamp, uint64_t *clock,
                               void *stream);

/* Copy the rows of flat ids ids[i] into slots slots[i] from the registered
 * sources (host arrays of `count` entries), without touching the slot table:
 * used to warm slots whose owners were set by oes_cache_set_state.  Same copy
 * kernel as copy_missing.  Errors: OES_ERR_ARG (range, missing source). */
oes_status oes_cache_load_rows(oes_cache *c, const int32_t *slots, const int64_t *ids,
                               int32_t count, void *stream);

/* Fill every byte of every slot bank with `value` (test sentinel). */
oes_status oes_cache_fill_slots(oes_cache *c, uint8_t value, void *stream);

/* Device base address and row bytes of slot bank `bank` (row s at base + s*row_bytes). */
oes_status oes_cache_slot_bank(const oes_cache *c, int32_t bank, void **dev_base,
                               int64_t *row_bytes);
/* Number of slots, and the cache's schema. */
oes_status oes_cache_info(const oes_cache *c, int32_t *num_slots, oes_schema *schema);

/* Miss list of the last ensure_experts: *count entries (slot, flat id) in
 * install order (ascending id), the list copy_missing consumes (benchmark
 * guide §4.1, §4.4: ensure_experts yields the missing experts, copy_missing
 * gathers them).  Copies at most `cap` entries.  Syncs. */
oes_status oes_cache_get_misses(oes_cache *c, int32_t *count, int32_t *slots, int64_t *ids,
                                int32_t cap, void *stream);
/* Counters since creation (benchmark guide §4.3: hits and misses of the
 * remap, bytes copied; §5.4: last_indices is num_indices, the misses fetched
 * by the last step, and last_missing_full is num_missing_full, its misses
 * before the hybrid cap).  Syncs. */
oes_status oes_cache_stats(oes_cache *c, oes_stats *out, void *stream);
/* Syncs `stream`, then returns and clears the sticky device error: OES_OK,
 * OES_ERR_CAPACITY (a step requested more distinct experts than slots) or
 * OES_ERR_ARG (a step held an id outside [0, E)). */
oes_status oes_cache_check(oes_cache *c, void *stream);

/* Options.  OES_OPT_FUSED_COPY: 1 (default) one launch gathers every bank;
 * 0 one launch per bank (the A/B path; default taken from env OES_FUSED_COPY
 * at creation).  OES_OPT_COPY_MODE: OES_COPY_ZERO (default) the gather
 * kernel reads mapped pinned memory; OES_COPY_SDMA copy_missing syncs the
 * stream, reads the miss list and issues one DMA copy per (miss, bank)
 * (default from env OES_COPY_MODE=zerocopy|sdma): the DMA engines need the
 * rows' addresses on the host, so in this A/B mode copy_missing is not
 * asynchronous - the one step call that waits for the GPU.  OES_OPT_COPY_BLOCKS: grid
 * size of the gather (0 = default).  OES_OPT_FFN_PATH: how expert_ffn runs
 * several tokens - OES_FFN_PER_PAIR one GEMV per (token, pair), OES_FFN_GROUPED
 * pairs grouped by slot so that each expert's rows are read once per call and
 * dotted with all its tokens, OES_FFN_AUTO (default) grouped when the repeats
 * expected of uniform top-k routing save at least 128 MB of weight reads.  One
 * token always takes the per-pair path.  The paths agree to within rounding. */
enum { OES_OPT_FUSED_COPY = 1, OES_OPT_COPY_MODE = 2, OES_OPT_COPY_BLOCKS = 3, OES_OPT_FFN_PATH = 4 };
enum { OES_COPY_ZERO = 0, OES_COPY_SDMA = 1 };
enum { OES_FFN_AUTO = 0, OES_FFN_PER_PAIR = 1, OES_FFN_GROUPED = 2 };
oes_status oes_cache_set_option(oes_cache *c, int32_t option, int64_t value);

/* ------------------------------------------------------------------ the step */

/* Router workspace bytes for n tokens, H hidden, E experts. */
oes_status oes_route_workspace(int32_t n, int32_t hidden, int32_t num_experts, int64_t *bytes);

/* Top-k routing: logits = x . Wg (bf16 inputs, fp32 sums), softmax over the E
 * experts, the k largest in descending order (equal logits: lower expert
 * first; a NaN logit ranks below every number), weights renormalised to sum
 * to 1 (the top-k of each MoE layer;
 * benchmark guide §4.3 routes bs * topk experts per step).
 *   x   [n, H] bf16 device, wg [H, E] bf16 device (row-major)
 *   ids [n, k] int32 device out, w [n, k] float device out
 *   logits [n, E] float device out, or NULL
 *   workspace: device, >= oes_route_workspace bytes, 16-byte aligned.
 * Limits: 1 <= k <= min(E, 32), E a multiple of 8 and <= 512, n >= 0. */
oes_status oes_route(const void *x, const void *wg, int32_t n, int32_t hidden,
                     int32_t num_experts, int32_t k, int32_t *ids, float *w, float *logits,
                     void *workspace, int64_t workspace_bytes, void *stream);

/* Top-k of given router logits [n, E] float device: the same softmax, top-k
 * and renormalisation as oes_route without the router matmul (the prefill
 * layer routes its tokens' given logits before the grouped FFN of the
 * streamed layer, architecture walk-through §5).  ids [n, k] int32, w [n, k]
 * float, device.  Limits: 1 <= E <= 512, 1 <= k <= min(E, 32), n >= 0.  Async. */
oes_status oes_route_logits(const float *logits, int32_t n, int32_t num_experts, int32_t k,
                            int32_t *ids, float *w, void *stream);

/* ensure_experts: global LRU remap of layer `layer`'s routed experts onto the
 * slot pool (benchmark guide §4.1, §4.3; architecture walk-through §5).
 *   ids [n, k] int32 device (expert index within the layer), slot_ids [n, k]
 *   int32 device out.
 * One workgroup does the whole remap on the device:
 *   U = sorted distinct flat ids layer*E + ids; resident ones are hits; the
 *   others are installed in ascending id order into the evictable slots (those
 *   not holding a member of U) ordered by (not empty, stamp, owner, slot);
 *   the clock advances and every slot holding a member of U is stamped; the
 *   miss list (slot, id) is kept for copy_missing; slot_ids[t, j] is the slot
 *   of ids[t, j].
 * Device-side failures (an id outside [0, E): OES_ERR_ARG; |U| > num_slots:
 * OES_ERR_CAPACITY) leave the slot table unchanged, write -1 to slot_ids,
 * empty the miss list, make the following copy_missing / expert_ffn of this
 * step no-ops, and are reported by the next syncing call (oes_cache_check).
 * Host-side errors: layer outside [0, L), n*k < 0 or > 65536, k < 1.
 * Async. */
oes_status oes_ensure_experts(oes_cache *c, int32_t layer, const int32_t *ids, int32_t n,
                              int32_t k, int32_t *slot_ids, void *stream);

/* ensure_experts_hybrid (benchmark guide §5.4): the same remap, except that only
 * the first `take` missing ids (ascending flat id) get slots and are listed for
 * copy_missing; the rest keep no slot, their entries of slot_ids are -1 (the
 * expert FFN skips them; they are the CPU executor's share) and they are not
 * stamped.  take = min(cap, misses, slots not holding a requested id), so a
 * hybrid step never fails for capacity.  cap = max_fetch when max_fetch >= 0
 * (hybrid_max_fetch); otherwise misses x min(1, fetch_fraction) rounded half to
 * even (in double) when fetch_fraction >= 0, where fetch_fraction is the
 * measured pcie_bw / cpu_bw split; otherwise 1 (no bandwidth profile).
 * oes_cache_stats reports last_indices (num_indices) and last_missing_full
 * (num_missing_full).  Errors as oes_ensure_experts, OES_ERR_CAPACITY excepted;
 * OES_ERR_ARG for a NaN fetch_fraction. */
oes_status oes_ensure_experts_hybrid(oes_cache *c, int32_t layer, const int32_t *ids, int32_t n,
                                     int32_t k, int32_t *slot_ids, int32_t max_fetch,
                                     double fetch_fraction, void *stream);

/* copy_missing: for every (slot, flat id) of the last miss list and every bank
 * b, copy row id % E of layer id / E's host bank b into slot row `slot` of
 * slot bank b (benchmark guide §4.1, §4.4: a per-bank index gather, fused
 * across banks in one launch).  Async in the default zero-copy mode; in the
 * OES_COPY_SDMA mode it syncs `stream` first (see oes_cache_set_option).  A
 * miss whose layer has no registered source for some bank is skipped and sets
 * OES_ERR_ARG in the sticky status. */
oes_status oes_copy_missing(oes_cache *c, void *stream);

/* Workspace bytes expert_ffn needs for n tokens with top-k. */
oes_status oes_expert_ffn_workspace(const oes_cache *c, int32_t n, int32_t k, int64_t *bytes);

/* expert_ffn: y[t] = sum_j w[t, j] * (Wd . (silu(Wg . x_t) * (Wu . x_t)))
 * computed on slot slot_ids[t, j] of the slot cache (architecture walk-through
 * §5: hits are computed from the slot cache).  Quantised banks are dequantised
 * in registers; sums are fp32; y is bf16 (round to nearest even).
 *   x [n, H] bf16 device, slot_ids [n, k] int32 device (-1 = skip the pair),
 *   w [n, k] float device, y [n, H] bf16 device out, workspace device.
 * Formats: OES_BF16, OES_FP8_BLOCK128, OES_NVFP4, OES_Q4_0 (decode).  Limits:
 * n * k <= 32768, k <= 32, H <= 16384.  A no-op when the last ensure_experts
 * failed on the device.  Async. */
oes_status oes_expert_ffn(oes_cache *c, const void *x, const int32_t *slot_ids, const float *w,
                          int32_t n, int32_t k, void *y, void *workspace, int64_t workspace_bytes,
                          void *stream);

/* expert_ffn for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results as oes_expert_ffn, with the workspace taken from a
 * library-owned device array of OES_FFN_NOALLOC_SCRATCH_BYTES per GPU (placed
 * with the library's device code on each GPU it runs on, held until the
 * process ends) instead of an argument.  Calls no hipMalloc / hipFree or other allocating routine.
 * Requires oes_expert_ffn_workspace(c, n, k) <= OES_FFN_NOALLOC_SCRATCH_BYTES
 * (about 2 n k I bytes for one token and 2 n k I + 4 n k (H + 3) for several:
 * n k <= 1720 at H = 2048, I = 768; n k <= 511 at H = 7168, I = 2048), else
 * OES_ERR_ARG with a message naming both sizes and nothing enqueued.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, or two caches on two threads) race on it and are not allowed;
 * calls ordered on one stream are fine (each call writes every workspace entry
 * it later reads).  Other arguments and errors as oes_expert_ffn.  Async. */
#define OES_FFN_NOALLOC_SCRATCH_BYTES (16 << 20)
oes_status oes_expert_ffn_noalloc(oes_cache *c, const void *x, const int32_t *slot_ids, const float *w,
                                  int32_t n, int32_t k, void *y, void *stream);

/* ------------------------------------------------------------------ prefill layer streaming */
/*
 * Whole-layer double-buffered streaming for prefill (architecture walk-through
 * §5): `depth` device buffers each hold every expert of one layer (row e =
 * expert e) for every bank.  oes_layers_prefetch copies layer l's host banks
 * into buffer l % depth on a copy stream with DMA and records an event;
 * oes_layers_ffn makes the compute stream wait for that event, runs the
 * grouped expert FFN of the layer on that buffer, and records a release event
 * the next prefetch into the same buffer waits for.
 */
typedef struct oes_layers oes_layers;

oes_status oes_layers_create(const oes_schema *schema, int32_t depth, int32_t device,
                             oes_layers **out);
oes_status oes_layers_destroy(oes_layers *p);
/* Same contract as oes_cache_set_source. */
oes_status oes_layers_set_source(oes_layers *p, int32_t bank, int32_t layer, const void *host,
                                 int64_t bytes);
/* Enqueue the copy of layer `layer` into buffer layer % depth on copy_stream. */
oes_status oes_layers_prefetch(oes_layers *p, int32_t layer, void *copy_stream);
/* Device address and bytes of bank `bank` in buffer `index`. */
oes_status oes_layers_buffer(const oes_layers *p, int32_t index, int32_t bank, void **dev,
                             int64_t *bytes);
/* Workspace bytes oes_layers_ffn needs for n tokens with top-k. */
oes_status oes_layers_ffn_workspace(const oes_layers *p, int32_t n, int32_t k, int64_t *bytes);
/* Grouped expert FFN of layer `layer` (which must have been prefetched) over
 * n tokens routed to ids [n, k] int32 device with weights w [n, k] float
 * device: y [n, H] bf16.  An id outside [0, E) (-1, say) skips its pair; a
 * token whose pairs are all skipped gets y = 0; n = 0 launches nothing.
 * Format: OES_MXFP4_T (MFMA grouped GEMM).  Async. */
oes_status oes_layers_ffn(oes_layers *p, int32_t layer, const void *x, const int32_t *ids,
                          const float *w, int32_t n, int32_t k, void *y, void *workspace,
                          int64_t workspace_bytes, void *compute_stream);

/* ------------------------------------------------------------------ measurement probes */
/* Ceilings the benchmark divides by.  All sync and return times in ms.
 * oes_probe_h2d_dma: one hipMemcpyAsync of `bytes` from pinned host to device.
 * oes_probe_h2d_kernel: the gather kernel's read of `bytes` of mapped pinned
 *   host memory into device memory (the zero-copy path's ceiling).
 * oes_probe_hbm_read: `count` streaming reads of `bytes` each, launched back to
 *   back, the i-th at dev + i * stride (a stride that walks past the 256 MB
 *   memory-side cache keeps every read cold); *ms is the time per read.  The
 *   caller's buffer spans (count - 1) * stride + bytes; bytes and stride are
 *   multiples of 16, count >= 1.
 * oes_probe_mfma_bf16: `blocks` workgroups of 4 waves, each wave `iters` rounds of
 *   4 independent v_mfma_f32_32x32x16_bf16 on register operands; `*flops`
 *   receives the dense flops issued.  `sink` is a device float the kernel may
 *   write (it never does in practice).  blocks >= 1, 1 <= iters <= 1 << 24.
 * oes_probe_mfma_f8f4: the same with v_mfma_scale_f32_32x32x64_f8f6f4, A e4m3 and
 *   B e2m1 with e8m0 block scales (the prefill GEMM's instruction). */
oes_status oes_probe_h2d_dma(void *dev, const void *host, int64_t bytes, void *stream, float *ms);
oes_status oes_probe_h2d_kernel(void *dev, const void *host, int64_t bytes, int32_t blocks,
                                void *stream, float *ms);
oes_status oes_probe_hbm_read(const void *dev, int64_t bytes, int64_t stride, int32_t count, void *sink,
                              void *stream, float *ms);
oes_status oes_probe_mfma_bf16(int32_t blocks, int32_t iters, void *sink, void *stream, float *ms,
                               double *flops);
oes_status oes_probe_mfma_f8f4(int32_t blocks, int32_t iters, void *sink, void *stream, float *ms,
                               double *flops);

/* ------------------------------------------------------------------ decoder check */
/* ---------------------------------------------------------------- hybrid backend
 * CPU MoE executor (FreeToken architecture walk-through §5: what PCIe cannot
 * bring in time is computed by the host cores with AVX-512 GEMVs; FreeToken
 * MoE benchmark guide §5.2-§5.4: ensure_experts_hybrid hands the experts above
 * the fetch cap (slot -1) to this executor).  Host code: every pointer below is
 * a host pointer, nothing touches the GPU, calls block until done.  Formats
 * with a CPU path: OES_BF16, OES_NVFP4, OES_Q4_0.  An executor is not
 * thread-safe: use it from one thread. */
typedef struct oes_cpu_moe oes_cpu_moe;

/* Create an executor for `schema` with `threads` worker threads (0: three
 * quarters of the CPUs the process may use - its affinity mask capped by a
 * cgroup CPU quota - which leaves room for the caller's other threads; the
 * calling thread is one of the workers).
 * Errors: OES_ERR_ARG (schema not from oes_schema_make, threads outside
 * [0, 1024]), OES_ERR_UNSUPPORTED (a format without a CPU path, or a host
 * without AVX-512 F/BW/VL/BF16 and F16C). */
oes_status oes_cpu_moe_create(const oes_schema *schema, int32_t threads, oes_cpu_moe **out);
oes_status oes_cpu_moe_destroy(oes_cpu_moe *m);
oes_status oes_cpu_moe_threads(const oes_cpu_moe *m, int32_t *threads);

/* Register bank `bank` of layer `layer`: E rows of row_bytes, expert-major,
 * the same host tensors a cache reads (any host memory; caller-owned, must
 * outlive the executor).  bytes must equal E * row_bytes.  Reads one byte of
 * every 4 KiB page (on the executor's threads), so that the first-touch
 * mapping of pinned pages happens here and not in a step.  Errors: OES_ERR_ARG. */
oes_status oes_cpu_moe_set_source(oes_cpu_moe *m, int32_t bank, int32_t layer, const void *host, int64_t bytes);

/* The CPU part of a hybrid step: for every pair (t, j) with slot_ids[t, j] < 0,
 * expert e = ids[t, j] of `layer`:
 *   h = silu(Wg_e . x_t) * (Wu_e . x_t)   (fp32, rounded to bf16)
 *   y[t] += w[t, j] * (Wd_e . h)           (fp32, pairs in (t, j) order)
 * y rows of tokens with no such pair are 0.  x bf16 [n, H], ids and slot_ids
 * int32 [n, k], w fp32 [n, k], y fp32 [n, H]; all host, row-major.  Results
 * do not depend on the thread count.  Errors: OES_ERR_ARG (range, an id of a
 * CPU pair outside [0, E), a bank of the layer without a source). */
oes_status oes_cpu_moe_run(oes_cpu_moe *m, int32_t layer, const void *x_bf16, const int32_t *ids,
                           const int32_t *slot_ids, const float *w, int32_t n, int32_t k, float *y);

/* DRAM read ceiling (benchmark guide §5.2: a STREAM-style read): every byte of
 * the host buffer read once by the executor's threads; *ms = wall time. */
oes_status oes_cpu_moe_probe_read(oes_cpu_moe *m, const void *buf, int64_t bytes, double *ms);

/* Backend decision of benchmark guide §5.2 and fetch split of §5.4:
 * *hybrid = 1 iff the format has a CPU path and cpu_gbps > threshold *
 * pcie_gbps (the page's default threshold is 2); *fetch_fraction = pcie_gbps /
 * cpu_gbps, or 1 when the CPU is no faster (the hybrid_fetch_fraction that
 * oes_ensure_experts_hybrid takes).  Errors: OES_ERR_ARG (pcie_gbps <= 0,
 * cpu_gbps < 0, threshold <= 0, NaN). */
oes_status oes_hybrid_decide(int32_t format, double cpu_gbps, double pcie_gbps, double threshold,
                             int32_t *hybrid, double *fetch_fraction);

/* One hybrid MoE layer step (benchmark guide §5.4, architecture walk-through
 * §5): oes_ensure_experts_hybrid with (max_fetch, fetch_fraction); the step's
 * x, ids, slot_ids and w copied to `host_ws`; copy_missing and expert_ffn
 * enqueued on `stream` (the GPU computes the fetched and resident experts,
 * skipping the -1 pairs); the host waits only for the small copies, then runs
 * oes_cpu_moe_run on the -1 pairs while the GPU copies and computes; the CPU
 * result goes to `dev_ws` and is added into y (oes_combine_cpu), after the FFN
 * in stream order.  Returns once the CPU part is done and the rest is
 * enqueued.  x bf16 [n, H], ids int32 [n, k], w fp32 [n, k], slot_ids int32
 * [n, k] (written), y bf16 [n, H] and the FFN workspace are device buffers as
 * for the separate calls; host_ws must be pinned host memory (hipHostMalloc /
 * torch pin_memory) of at least the size oes_hybrid_workspace gives, dev_ws
 * device memory of its size; both are reused by the next step on the same
 * stream.  `cpu` must have the cache's schema and sources.  Errors: those of
 * the calls it makes, OES_ERR_ARG (workspace sizes, schema mismatch). */
oes_status oes_hybrid_workspace(const oes_cache *c, int32_t n, int32_t k, int64_t *host_bytes, int64_t *dev_bytes);
oes_status oes_hybrid_step(oes_cache *c, oes_cpu_moe *cpu, int32_t layer, const void *x, const int32_t *ids,
                           const float *w, int32_t n, int32_t k, int32_t *slot_ids, void *y, void *ffn_ws,
                           int64_t ffn_ws_bytes, void *host_ws, int64_t host_ws_bytes, void *dev_ws,
                           int64_t dev_ws_bytes, int32_t max_fetch, double fetch_fraction, void *stream);

/* y_bf16[i] = bf16_rne(float(y_bf16[i]) + y_cpu[i]) for i < count: adds the
 * executor's output (copied to the device) into the GPU FFN's output of the
 * same step.  Device pointers; enqueued on `stream`. */
oes_status oes_combine_cpu(void *y_bf16, const float *y_cpu, int64_t count, void *stream);

/* Decode `n` elements of type `elem` (OES_ELEM_E4M3, OES_ELEM_FP4X2,
 * OES_ELEM_E8M0, OES_ELEM_BF16, OES_ELEM_FP16, OES_ELEM_Q4X2) from device
 * `codes` into device float `out` with the same device routines the FFN
 * kernels use (FP4X2: two elements per byte, element 2j in the low nibble;
 * Q4X2: n a multiple of 32, GGUF Q4_0 nibble order, output q - 8 before the
 * block scale).  Async.  For tests. */
oes_status oes_debug_decode(int32_t elem, const void *codes, int32_t n, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* OES_H_ */
