// Prefill grouped expert FFN over a streamed layer buffer: MXFP4 weights on the
// gfx950 block-scaled MFMA.
//
// FreeToken architecture walk-through §5: prefill streams whole layers through a
// double buffer; the FFN of a layer runs on the buffer holding it (row e =
// expert e).  FreeToken MoE benchmark guide §4.2: the MXFP4 format keeps six
// transposed banks - _blocks, _scales, _bias for gate_up and for down.
//
// Four launches (permute and split share the first):
//   permute    - one workgroup counts the (token, pair) routes per expert, scans
//                the counts into offsets and scatters the pair indices into
//                expert order (perm).  The order inside an expert does not
//                change any result: every output row of a GEMM is computed on
//                its own, with the same k order.  It also records each pair's
//                position in expert order (pos) and ranks the experts by row
//                count, largest first, for the GEMMs' dispatch order.
//   split      - the bf16 activations x become two e4m3 code planes, hi and lo,
//                with one power-of-two scale per 32-element block (below).
//   gemm<0>    - per expert e: h = silu(X_e Wg_e^T + bg) * (X_e Wu_e^T + bu),
//                rounded to bf16 and split like x, X_e the gathered activation
//                rows of the pairs routed to e.
//   gemm<1>    - per expert e: o = h_e Wd_e^T + bd, rounded to bf16 (as h is
//                between the GEMMs), rows in expert order.
//   combine    - y_t = sum_j w[t, j] * o_{t,j} in pair order, bf16, each pair's
//                row found through its expert-order position (pos).
//
// Exact two-plane activations.  The weights stay MXFP4 (e2m1 codes with an e8m0
// scale per 32 k) and go to v_mfma_scale_f32_32x32x64_f8f6f4 as they are, with
// no conversion.  The activations are bf16 (8 significant bits); the MFMA's
// other operand takes e4m3 (4 significant bits) with an e8m0 scale per 32 k.
// Each 32-element block of a bf16 row is written as v = hi * 2^s + lo * 2^(s-4):
// s puts the block's largest magnitude in [2^7, 2^8), hi is v / 2^s rounded to
// e4m3, and the remainder (v / 2^s - hi) * 16 has at most 4 significant bits
// and lies below 2^8, so lo holds it exactly.  The split is exact for every
// element within 2^13 of its block's largest (smaller ones keep an error below
// 2^-20 of that largest), so the two MFMAs per product compute what a bf16 x
// fp4 product computes, with fp32 accumulation.  On gfx950 the fp8 x fp4 form
// issues at twice the bf16 MFMA's flop rate, so the pair costs no more than
// one bf16 MFMA over the same k, and the weights need no fp4 -> bf16 step.
//
// GEMM tiling (details at the kernel):
//   block = (expert, 128 / 256 output features) x all rows of the expert in
//   passes of 96; in gate_up, wave w owns 32 features (those 32 gate rows and
//   the matching 32 up rows, so silu(g) * u is formed in registers).  K runs in
//   quads of four 32-element MXFP4 blocks, each quad in two 64-k MFMA steps.
//   The A chunk of a quad (hi and lo codes and the row's four scale bytes) is
//   staged in LDS from registers loaded one quad ahead; the B operand needs no
//   LDS: the K-block-major layout [K/32][N][16 B] gives each lane the 16 bytes
//   of one MXFP4 block, which is its whole operand of one MFMA step.
//   Blocks are mapped XCD-aware: hardware deals consecutive block indices to
//   the 8 XCDs in turn, so block b runs on XCD b % 8; the experts of ranks r
//   with r % 8 == x are given to XCD x, which keeps an expert's activation rows
//   in one L2 while all its feature tiles stream their weights.  Ranks follow
//   row count, largest first: the longest blocks start first on every XCD, and
//   the tail of the launch holds the shortest ones.

#include <math.h>

#include <algorithm>

#include "oes_internal.h"

namespace oes {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;  // a global-memory u32x4

constexpr int kThreads = 256;
constexpr int BM = 96;             // rows per pass: three 32-row m-tiles
constexpr int LDA = 256 + 16;      // LDS bytes per A row of one quad: 128 hi codes, 128 lo codes, 16 pad
constexpr int kXcds = 8;
constexpr int kProbeChains = 4;    // accumulator chains per wave of the MFMA ceiling probes
constexpr int kMaxKb = 96;         // K / 32 limit of the grouped GEMM (K <= 3072)
constexpr int kLoShift = 4;        // lo plane scale = hi plane scale / 2^4
constexpr int kFmtE4m3 = 0, kFmtE2m1 = 4;  // operand formats of the block-scaled MFMA
static_assert(kThreads == 256, "sixteen A pieces per row: 16 rows per thread group pass");

struct GemmArgs {
  int32_t H, I, E, k, nk;
  int32_t ntiles;        // feature tiles per expert
  int32_t xcd;           // 1: XCD-aware block mapping (E % 8 == 0)
  const uint8_t *ahi;    // this phase's A: e4m3 hi codes [rows, K]
  const uint8_t *alo;    // e4m3 lo codes [rows, K]
  const uint8_t *asc;    // hi scale bytes [rows, kb4(K)] (lo scale = hi - 4)
  const int32_t *offsets;  // [E + 1]
  const int32_t *perm;     // [nk] pair indices in expert order
  const int32_t *order;    // [E] experts in dispatch order
  const uint8_t *blocks;   // this phase's _blocks bank, expert stride blocks_stride
  const uint8_t *scales;   // this phase's _scales bank
  const uint16_t *bias;    // this phase's _bias bank (bf16)
  int64_t blocks_stride, scales_stride, bias_stride;
  const u32x4 *zero16;   // 16 zero bytes: the source of A pieces past K
  uint8_t *hhi, *hlo;    // gate_up output h: e4m3 planes [nk, I], expert order
  uint8_t *hsc;          // its hi scale bytes [nk, kb4(I)]
  uint16_t *obuf;        // [nk, H] bf16, expert order
};

// scale bytes per row of a split plane: K / 32 rounded up to whole quads of four
__host__ __device__ inline int kb4_of(int K) { return ((K / 32) + 3) & ~3; }

__device__ inline float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ inline uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two-plane split of one bf16 value v held by lane (c, half) of a 32-lane half
// whose lanes hold the 32 elements of one block: every lane of the wave must
// call it together (the block's largest magnitude is reduced over the half).
// hi / lo are e4m3 codes, sbyte the hi plane's e8m0 scale byte, kept in
// [4, 250] so that the lo scale sbyte - 4 is a finite e8m0 value too.
struct Split {
  uint32_t hi, lo, sbyte;
};
__device__ __forceinline__ Split split_e4m3(float v) {
  // block maximum of |v| (as non-negative int bits): a max-scan along each
  // 16-lane row by DPP row shifts (lanes shifted in from outside the row read
  // 0, which never wins), after which lane 15 of a row holds the row's maximum;
  // the four row maxima are read into scalars and each half-wave takes the
  // larger of its two rows
  int m = (int)(__float_as_uint(v) & 0x7fffffffu);
  m = max(m, __builtin_amdgcn_mov_dpp(m, 0x111, 0xf, 0xf, true));  // row_shr:1
  m = max(m, __builtin_amdgcn_mov_dpp(m, 0x112, 0xf, 0xf, true));  // row_shr:2
  m = max(m, __builtin_amdgcn_mov_dpp(m, 0x114, 0xf, 0xf, true));  // row_shr:4
  m = max(m, __builtin_amdgcn_mov_dpp(m, 0x118, 0xf, 0xf, true));  // row_shr:8
  const int lo_half = max(__builtin_amdgcn_readlane(m, 15), __builtin_amdgcn_readlane(m, 31));
  const int hi_half = max(__builtin_amdgcn_readlane(m, 47), __builtin_amdgcn_readlane(m, 63));
  const uint32_t a = (uint32_t)((threadIdx.x & 32) ? hi_half : lo_half);
  const uint32_t sb = (uint32_t)min(max((int)(a >> 23) - 7, 4), 250);
  const float xs = v * __uint_as_float((254u - sb) << 23);  // v / 2^(sb - 127), exact
  const uint32_t hp = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(xs, 0.f, 0, false);
  const float hf = __builtin_amdgcn_cvt_f32_fp8((int)hp, 0);
  const uint32_t lp = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((xs - hf) * 16.f, 0.f, 0, false);
  return {hp & 0xffu, lp & 0xffu, sb};
}

// 4x4 byte transpose inside each quad of lanes: lane c (= lane % 4) of the quad
// passes p, whose byte r belongs to row r; it receives the bytes c of the four
// lanes' p, lane c' in byte c'.
__device__ __forceinline__ uint32_t quad_transpose(uint32_t p, int c) {
  const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0xb1, 0xf, 0xf, false);  // quad_perm 1,0,3,2
  const uint32_t p2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0x4e, 0xf, 0xf, false);  // quad_perm 2,3,0,1
  const uint32_t p3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0x1b, 0xf, 0xf, false);  // quad_perm 3,2,1,0
  const int sh = 8 * c;
  return (((p >> sh) & 0xffu) << (8 * c)) | (((p1 >> sh) & 0xffu) << (8 * (c ^ 1))) |
         (((p2 >> sh) & 0xffu) << (8 * (c ^ 2))) | (((p3 >> sh) & 0xffu) << (8 * (c ^ 3)));
}

// ------------------------------------------------------------------ permute
// Run by one workgroup of 1024 threads.
__device__ __forceinline__ void permute_body(const int32_t *ids, int nk, int E, int32_t *offsets, int32_t *perm,
                                             int32_t *pos, int32_t *order, uint32_t *zeros) {
  if (threadIdx.x < 64) zeros[threadIdx.x] = 0u;  // the GEMMs' 256-byte zero source
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
    int at = -1;
    if (e >= 0 && e < E) {
      at = atomicAdd(&cursor[e], 1);
      perm[at] = p;
    }
    pos[p] = at;  // the pair's row in expert order (-1: skipped)
  }
  // dispatch order of the GEMMs: experts by row count, largest first (ties: lower
  // index first), so the longest blocks start first; identity past 1024 experts.
  // Expert e's rank (the experts that come before it) is counted by 1024 / E
  // threads over slices of the counts; cursor holds their partial counts.
  __syncthreads();  // the scatter is done with cursor
  if (E <= 1024) {
    const int parts = 1024 / E;
    if ((int)threadIdx.x < E * parts) {
      const int e = threadIdx.x % E, part = threadIdx.x / E;
      const int c = hist[e];
      int cnt = 0;
      for (int q = E * part / parts; q < E * (part + 1) / parts; ++q) cnt += (hist[q] > c) || (hist[q] == c && q < e);
      cursor[threadIdx.x] = cnt;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      int rank = 0;
      for (int part = 0; part < parts; ++part) rank += cursor[part * E + e];
      order[rank] = e;
    }
  } else {
    for (int e = threadIdx.x; e < E; e += blockDim.x) order[e] = e;
  }
}

// ------------------------------------------------------------------ split
// x [rows, K] bf16 -> hi / lo e4m3 planes [rows, K] and hi scale bytes
// [rows, kb4(K)], the same two-plane split as split_e4m3 with eight elements
// per lane: four lanes hold a 32-element block (K % 64 == 0, so blocks never
// straddle rows and count = rows * K is a multiple of 32: each group of four
// lanes is wholly in or out).  The scale bytes past K / 32 (up to the quad) get
// 127 (scale 1): the GEMMs multiply them by zero codes only.
// Lane `lane` (of the whole launch's split lanes) takes elements 8 lane .. 8 lane + 7.
__device__ __forceinline__ void split_body(const uint16_t *x, int64_t count, int K, uint8_t *hi, uint8_t *lo,
                                           uint8_t *sc, int64_t lane) {
  const int64_t i = lane * 8;
  if (i >= count) return;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + i));
  float f[8];
  uint32_t a = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(v[j] << 16);
    f[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    a = max(a, max(__float_as_uint(f[2 * j]) & 0x7fffffffu, __float_as_uint(f[2 * j + 1]) & 0x7fffffffu));
  }
  a = max(a, (uint32_t)__shfl_xor((int)a, 1));
  a = max(a, (uint32_t)__shfl_xor((int)a, 2));
  const uint32_t sb = (uint32_t)min(max((int)(a >> 23) - 7, 4), 250);
  const float inv = __uint_as_float((254u - sb) << 23);
  u32x2 hv, lv;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const float x0 = f[4 * w] * inv, x1 = f[4 * w + 1] * inv, x2 = f[4 * w + 2] * inv, x3 = f[4 * w + 3] * inv;
    int hp = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    hp = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hp, true);
    const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hp, false);
    const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hp, true);
    int lp = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - h01[0]) * 16.f, (x1 - h01[1]) * 16.f, 0, false);
    lp = __builtin_amdgcn_cvt_pk_fp8_f32((x2 - h23[0]) * 16.f, (x3 - h23[1]) * 16.f, lp, true);
    hv[w] = (uint32_t)hp;
    lv[w] = (uint32_t)lp;
  }
  *reinterpret_cast<u32x2 *>(hi + i) = hv;
  *reinterpret_cast<u32x2 *>(lo + i) = lv;
  const int64_t row = i / K;
  const int col = (int)(i - row * K);
  const int nkb = K / 32, kb4 = kb4_of(K);
  if ((col & 31) == 0) sc[row * kb4 + col / 32] = (uint8_t)sb;
  if (col == 0)
    for (int j = nkb; j < kb4; ++j) sc[row * kb4 + j] = 127;
}

// ------------------------------------------------------------------ prep
// permute and split are independent: one launch runs both, block 0 permuting the
// pairs while blocks 1.. split x, so the single-workgroup permute hides behind
// the split instead of adding its time.
struct PrepArgs {
  const int32_t *ids;
  int nk, E;
  int32_t *offsets, *perm, *pos, *order;
  uint32_t *zeros;
  const uint16_t *x;
  int64_t count;
  int K;
  uint8_t *hi, *lo, *sc;
};
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepArgs a) {
  if (blockIdx.x == 0)
    permute_body(a.ids, a.nk, a.E, a.offsets, a.perm, a.pos, a.order, a.zeros);
  else
    split_body(a.x, a.count, a.K, a.hi, a.lo, a.sc, (int64_t)(blockIdx.x - 1) * kPrepThreads + threadIdx.x);
}

// ------------------------------------------------------------------ grouped GEMM
// Block = (expert, feature tile), 4 waves; rows of the expert in passes of at
// most BM = 96, each pass run by a body specialised on its count of 32-row
// m-tiles so that its quad loop has no branches.
//
// v_mfma_scale_f32_32x32x64_f8f6f4, A e4m3 and B e2m1 (lane layout checked on
// the GPU with an in-bounds probe): in lane l = (c, h) with c = l % 32 and
// h = l / 32, B is column c, k = 32h + i for code i of the lane's 16 bytes
// (low nibble first), with the lane's scale byte; A is row c, bytes 0..15 at
// k = 16h + i and bytes 16..31 at k = 32 + 16h + i, and the scale byte of lane
// (c, h) scales A's k-block h (k = 32h .. 32h + 31).  D element r of lane l is
// row 4h + (r % 4) + 8(r / 4), column c.
//
// K order.  Step j (0, 1) of quad q covers MXFP4 blocks kb0 = 4q + 2j and
// kb0 + 1: lane (n, h) of a weight tile loads the 16 bytes at (kb0 + h, n) of
// the [K/32][N][16] bank, which is its whole B operand; lane (m, h) of the A
// side reads its 2 x 16 bytes of each plane from the staged row.
//
// Pipelining.  The block's weight scale bytes (its 256 weight rows x K/32
// blocks) are copied to LDS once.  B: each wave holds one quad's two steps per
// n-tile in registers; step j of quad q + 1 is loaded as soon as quad q's MFMAs
// of step j are issued.  A: the chunk of quad q + 1 (the pass's rows x 128 k of
// both planes, and each row's four scale bytes) is loaded into registers while
// quad q is multiplied from LDS, then stored to the other LDS buffer; one
// barrier per quad.  The steady-state loop has no conditions, so the
// compiler's memory-counter waits stay exact.  Indexes past the data are
// clamped (B) or pointed at a zero block (A, k past K), never branched on; the
// A scale bytes past K / 32 are finite, so those steps add exact zeros.  Each
// output row of an MFMA depends only on its own A row, so A rows past the
// pass's last row may hold anything: their outputs are never stored.
//
// Each wave owns two 32-feature n-tiles: gate_up - the gate tile and the up
// tile of the same 32 features (128 features per block); down - two consecutive
// tiles (256 features per block).  Tiles past the last feature run on clamped
// rows and are not stored.
constexpr int kUnroll = 2;  // quads per steady-state iteration: the LDS buffer parity is static
constexpr int NTW = 2;
constexpr int kRowsB = 256;  // weight rows per block

struct Tile {
  int e, off, m0, mrows;
  int K, N, nkb, nq, kb4;
  int nrow[NTW], f[NTW], lrow[NTW];
  bool tile_on[NTW];
  int n32, h;
};

template <int PHASE, int MT>
__device__ __forceinline__ void gemm_pass(const GemmArgs &g, const Tile &T, uint8_t (*As)[BM * LDA],
                                          uint32_t (*Asc)[kThreads], const int32_t *rowidx,
                                          const uint8_t *sc_lds) {
  constexpr int AP = 2 * MT;  // 16-byte A pieces per thread per quad
  const uint8_t *blk = g.blocks + (int64_t)T.e * g.blocks_stride;
  const int n32 = T.n32, h = T.h;
  // A piece: row 16i + rsub, 16 bytes at c16 * 16 of the staged row (hi plane for
  // c16 < 8, lo plane for c16 >= 8)
  const int c16 = threadIdx.x & 15, rsub = threadIdx.x >> 4;
  const uint8_t *psrc = (c16 < 8 ? g.ahi : g.alo) + (c16 & 7) * 16;

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  // A rows: rowidx < 0 marks a row past the pass (read row 0 instead)
  uint32_t aoff[AP];
#pragma unroll
  for (int i = 0; i < AP; ++i) aoff[i] = (uint32_t)max(rowidx[16 * i + rsub], 0) * (uint32_t)T.K;
  // thread t also stages the four scale bytes per quad of row min(t, BM - 1)
  // (the m-tiles read those of rows below 32 * MT); no thread is left out, so
  // the staging has no branch
  const uint8_t *ssrc = g.asc + (uint32_t)max(rowidx[min((int)threadIdx.x, BM - 1)], 0) * (uint32_t)T.kb4;
  // pieces past K read the zero block: a select on the loaded value would make
  // the wave wait for the loads at once instead of at the quad's end
  const uint64_t zero_addr = reinterpret_cast<uint64_t>(g.zero16);
  u32x4 areg[AP];
  uint32_t sreg;
  auto load_a = [&](int q) {
    const int k0 = q * 128;
    const bool kin = k0 + (c16 & 7) * 16 < T.K;
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      uint64_t src = kin ? reinterpret_cast<uint64_t>(psrc + aoff[i] + k0) : zero_addr;
      asm volatile("" : "+v"(src));  // keep the select on the address
      // every feature-tile block of the expert reads these rows: keep them in L2
      // (the weights, read once, are loaded non-temporal)
      areg[i] = *reinterpret_cast<const gu32x4 *>(src);
    }
    sreg = *reinterpret_cast<const uint32_t *>(ssrc + 4 * q);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AP; ++i) *reinterpret_cast<u32x4 *>(&As[buf][(16 * i + rsub) * LDA + c16 * 16]) = areg[i];
    Asc[buf][threadIdx.x] = sreg;
  };
  // B: one quad's two steps; step j of quad q + 1 is loaded as soon as quad q's
  // MFMAs of step j are issued
  u32x4 bw[2][NTW];
  const int64_t kstride = (int64_t)T.N * 16;
  uint32_t boff[NTW], soff[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    boff[t] = (uint32_t)(T.nrow[t] * 16 + h * T.N * 16);
    soff[t] = (uint32_t)(h * kRowsB + T.lrow[t]);
  }
  auto step_kb0 = [&](int j, int q) { return min(4 * q + 2 * j, T.nkb - 2); };
  auto load_b = [&](int j, int q) {
    const uint8_t *ub = blk + (int64_t)step_kb0(j, q) * kstride;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      bw[j][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ub + boff[t]));
  };

  // one 64-k step: per m-tile, the hi plane's MFMAs on both n-tiles, then the lo plane's
  auto step = [&](int j, int q, const uint8_t *Ab, const uint32_t *sdw) {
    const uint8_t *sl = sc_lds + step_kb0(j, q) * kRowsB;
    int sbv[NTW];
    i32x8 bop[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      sbv[t] = sl[soff[t]];
      bop[t] = i32x8{(int)bw[j][t][0], (int)bw[j][t][1], (int)bw[j][t][2], (int)bw[j][t][3], 0, 0, 0, 0};
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t *ar = Ab + (mt * 32 + n32) * LDA + 64 * j + 16 * h;
      const u32x4 h0 = *reinterpret_cast<const u32x4 *>(ar), h1 = *reinterpret_cast<const u32x4 *>(ar + 32);
      const u32x4 l0 = *reinterpret_cast<const u32x4 *>(ar + 128), l1 = *reinterpret_cast<const u32x4 *>(ar + 160);
      const int sah = (int)((sdw[mt] >> (8 * (2 * j + h))) & 0xffu);
      const int sal = sah - kLoShift;
      const i32x8 ahi = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
      const i32x8 alo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[mt][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ahi, bop[t], acc[mt][t], kFmtE4m3, kFmtE2m1, 0,
                                                                     sah, 0, sbv[t]);
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[mt][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo, bop[t], acc[mt][t], kFmtE4m3, kFmtE2m1, 0,
                                                                     sal, 0, sbv[t]);
    }
  };

  // full: both steps (the steady state); otherwise the second step runs only
  // where its blocks exist (the last quad of a K that is an odd count of 64)
  // a quad's loads and MFMAs are issued at raised wave priority, lowered again
  // for the barrier, so that of the two waves sharing a SIMD the one still
  // working keeps the matrix pipe fed while the other waits
  auto quad = [&](int q, bool more, bool full) {
    __builtin_amdgcn_s_setprio(1);
    if (more) load_a(q + 1);
    const uint8_t *Ab = As[q & 1];
    uint32_t sdw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sdw[mt] = Asc[q & 1][mt * 32 + n32];
    step(0, q, Ab, sdw);
    load_b(0, q + 1);
    if (full || 4 * q + 2 < T.nkb) step(1, q, Ab, sdw);
    load_b(1, q + 1);
    if (more) store_a((q + 1) & 1);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  };

  load_b(0, 0);
  load_b(1, 0);
  load_a(0);
  store_a(0);
  __syncthreads();
  // steady state: every quad of the group has a successor
  int q0 = 0;
  for (; q0 + kUnroll < T.nq; q0 += kUnroll) {
#pragma unroll
    for (int d = 0; d < kUnroll; ++d) quad(q0 + d, true, true);
  }
  // the last one to kUnroll quads
#pragma unroll
  for (int d = 0; d < kUnroll; ++d)
    if (q0 + d < T.nq) quad(q0 + d, q0 + d + 1 < T.nq, false);

  // epilogue: acc[mt][t][r] is row mt*32 + 4h + (r%4) + 8(r/4) of the pass, feature f[t]
  const uint16_t *bias = g.bias + (int64_t)T.e * g.bias_stride;
  if (PHASE == 0) {
    if (T.tile_on[0]) {  // uniform over the wave: the split reduces over lanes
      const float bg = bf16f(bias[T.f[0]]), bu = bf16f(bias[g.I + T.f[0]]);
      const int kb4 = kb4_of(g.I), nkb = g.I / 32;
      const int fb = T.f[0] / 32;  // this wave's 32 features are one k-block of down
      // lane quad (4q .. 4q + 3) holds rows m .. m + 3 (r = 4rq + 0..3) of features
      // 4q .. 4q + 3; after a 4x4 byte transpose inside the quad, lane c holds the
      // four features of row m + c as one dword
      const int c = n32 & 3;
      const int fcol = T.f[0] & ~3;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          uint32_t ph = 0, pl = 0, sc = 0;
#pragma unroll
          for (int r3 = 0; r3 < 4; ++r3) {
            const int r = 4 * rq + r3;
            const float gv = acc[mt][0][r] + bg, uv = acc[mt][1][r] + bu;
            // silu(g) * u with the hardware reciprocal (about 1 ulp; h is rounded to
            // bf16 next, by the hardware conversion, round to nearest even)
            const float hv = (float)(__bf16)(gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv);
            const Split s = split_e4m3(hv);
            ph |= s.hi << (8 * r3);
            pl |= s.lo << (8 * r3);
            sc = r3 == c ? s.sbyte : sc;
          }
          const uint32_t th = quad_transpose(ph, c), tl = quad_transpose(pl, c);
          const int m = mt * 32 + 4 * h + 8 * rq + c;
          if (m < T.mrows) {
            const int64_t row = T.off + T.m0 + m;
            *reinterpret_cast<uint32_t *>(g.hhi + row * g.I + fcol) = th;
            *reinterpret_cast<uint32_t *>(g.hlo + row * g.I + fcol) = tl;
            if (n32 < 4) {  // one lane per row writes its scale byte (and the pad past K / 32)
              g.hsc[row * kb4 + fb] = (uint8_t)sc;
              if (fb == nkb - 1)
                for (int j = nkb; j < kb4; ++j) g.hsc[row * kb4 + j] = 127;
            }
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
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mt * 32 + 4 * h + (r & 3) + 8 * (r >> 2);
          if (m < T.mrows)
            g.obuf[(int64_t)(T.off + T.m0 + m) * g.H + T.f[t]] =
                __builtin_bit_cast(uint16_t, (__bf16)(acc[mt][t][r] + bd));
        }
      }
    }
  }
}

template <int PHASE>
__global__ __launch_bounds__(kThreads, 2) void moe_gemm_kernel(GemmArgs g) {
  constexpr int NFB = PHASE == 0 ? 128 : 256;  // features per block
  __shared__ __align__(16) uint8_t As[2][BM * LDA];
  __shared__ uint32_t Asc[2][kThreads];
  __shared__ int32_t rowidx[BM];
  __shared__ __align__(16) uint8_t sc_lds[kMaxKb * kRowsB];
  Tile T;
  int nt;
  int rank;
  if (g.xcd) {
    const int x = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
    rank = x + kXcds * (local / g.ntiles);
    nt = local % g.ntiles;
  } else {
    rank = blockIdx.x / g.ntiles;
    nt = blockIdx.x % g.ntiles;
  }
  if (rank >= g.E) return;
  T.e = g.order[rank];
  T.off = g.offsets[T.e];
  const int m_e = g.offsets[T.e + 1] - T.off;
  if (m_e <= 0) return;
  T.K = PHASE == 0 ? g.H : g.I;
  T.N = PHASE == 0 ? 2 * g.I : g.H;
  const int nfeat = PHASE == 0 ? g.I : g.H;
  T.nkb = T.K / 32;
  T.nq = (T.nkb + 3) >> 2;
  T.kb4 = kb4_of(T.K);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  T.n32 = lane & 31;
  T.h = lane >> 5;
  if (PHASE == 0) {
    const int fbase = nt * NFB + wave * 32;
    T.f[0] = T.f[1] = fbase + T.n32;
    T.nrow[0] = min(T.f[0], g.I - 1);
    T.nrow[1] = g.I + T.nrow[0];
    T.lrow[0] = wave * 32 + T.n32;
    T.lrow[1] = 128 + T.lrow[0];
    T.tile_on[0] = T.tile_on[1] = fbase < nfeat;
  } else {
    const int fbase = nt * NFB + wave * 64;
    T.f[0] = fbase + T.n32;
    T.f[1] = T.f[0] + 32;
    T.nrow[0] = min(T.f[0], T.N - 1);
    T.nrow[1] = min(T.f[1], T.N - 1);
    T.lrow[0] = wave * 64 + T.n32;
    T.lrow[1] = T.lrow[0] + 32;
    T.tile_on[0] = fbase < nfeat;
    T.tile_on[1] = fbase + 32 < nfeat;
  }
  // scale bytes of the block's 256 weight rows: sc_lds[kb][local row], taken as
  // dwords of four rows (rows past the matrix clamp to its last dword; their
  // tiles are never stored).  Thread (w, c) copies dword c of blocks w, w + 4,
  // ..., w + 92: every load is issued before the first LDS write, so the staging
  // costs one memory round trip instead of one per dword.  Blocks past K / 32
  // get copies of the last block (the array holds kMaxKb of them; the quad loop
  // clamps its block index below K / 32, so they are never read).
  {
    constexpr int kScPer = kMaxKb * (kRowsB / 4) / kThreads;  // dwords per thread at most
    static_assert(kRowsB / 4 == 64 && kThreads == 256, "a wave copies one scale block row per step");
    const int r4 = lane * 4;
    int row;
    if (PHASE == 0) row = r4 < 128 ? min(nt * 128 + r4, g.I - 4) : g.I + min(nt * 128 + r4 - 128, g.I - 4);
    else row = min(nt * 256 + r4, T.N - 4);
    const uint8_t *scl = g.scales + (int64_t)T.e * g.scales_stride + row;
    uint32_t sv[kScPer];
#pragma unroll
    for (int u = 0; u < kScPer; ++u) {
      const int kb = min(wave + 4 * u, T.nkb - 1);
      sv[u] = *reinterpret_cast<const uint32_t *>(scl + (int64_t)kb * T.N);
    }
#pragma unroll
    for (int u = 0; u < kScPer; ++u) *reinterpret_cast<uint32_t *>(&sc_lds[(wave + 4 * u) * kRowsB + r4]) = sv[u];
  }

  for (T.m0 = 0; T.m0 < m_e; T.m0 += BM) {
    T.mrows = min(BM, m_e - T.m0);
    __syncthreads();  // the previous pass is done with rowidx and As; sc_lds is written
    for (int r = threadIdx.x; r < BM; r += kThreads) {
      int32_t o = -1;
      if (r < T.mrows) o = PHASE == 0 ? g.perm[T.off + T.m0 + r] / g.k : T.off + T.m0 + r;
      rowidx[r] = o;
    }
    __syncthreads();
    switch ((T.mrows + 31) >> 5) {
      case 1: gemm_pass<PHASE, 1>(g, T, As, Asc, rowidx, sc_lds); break;
      case 2: gemm_pass<PHASE, 2>(g, T, As, Asc, rowidx, sc_lds); break;
      default: gemm_pass<PHASE, 3>(g, T, As, Asc, rowidx, sc_lds); break;
    }
  }
}

// ------------------------------------------------------------------ MFMA ceilings
// Four independent accumulator chains per wave with operands in registers; the
// result is stored only on an impossible value, which keeps the chains live.
// bf16: v_mfma_f32_32x32x16_bf16.  f8f4: v_mfma_scale_f32_32x32x64_f8f6f4 with
// A e4m3 and B e2m1, the grouped GEMM's instruction.
template <bool F8F4>
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float *sink, int scale) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  i32x8 qa, qb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
    qa[i] = 0x30303030 + lane + i;
    qb[i] = i < 4 ? 0x21212121 + lane : 0;
  }
  const int sc = scale + (lane & 1);
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = (float)(c + r);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) {
      if (F8F4)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qb, acc[c], kFmtE4m3, kFmtE2m1, 0, sc, 0, sc);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) t += acc[c][0] + acc[c][15];
  if (t == 1234.5678f) sink[0] = t;
}

// ------------------------------------------------------------------ combine
// y[t, c..c+3] = sum_j w[t, j] * o[pos[t*k + j], c..c+3] (o bf16 in expert order, the
// sum in fp32), pairs with an invalid id skipped.
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t *obuf, const int32_t *pos, const int32_t *ids,
                                                           const float *w, int n, int k, int H, int E, uint16_t *y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * kThreads + threadIdx.x) * 4;
  if (t >= n || c >= H) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const float wj = w[p];
    const u32x2 ob = *reinterpret_cast<const u32x2 *>(obuf + (int64_t)pos[p] * H + c);
    const f32x4 o = {__uint_as_float(ob[0] << 16), __uint_as_float(ob[0] & 0xffff0000u), __uint_as_float(ob[1] << 16),
                     __uint_as_float(ob[1] & 0xffff0000u)};
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
  int64_t offsets, order, zeros, perm, pos, xhi, xlo, xsc, hhi, hlo, hsc, obuf, total;
};

WsLayout ws_layout(int H, int I, int n, int k, int E) {
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  WsLayout L;
  const int64_t nk = (int64_t)n * k;
  L.offsets = 0;
  L.order = up(4ll * (E + 1));
  L.zeros = L.order + up(4ll * E);
  L.perm = L.zeros + 256;
  L.pos = L.perm + up(4 * nk);
  L.xhi = L.pos + up(4 * nk);
  L.xlo = L.xhi + up((int64_t)n * H);
  L.xsc = L.xlo + up((int64_t)n * H);
  L.hhi = L.xsc + up((int64_t)n * kb4_of(H));
  L.hlo = L.hhi + up(nk * I);
  L.hsc = L.hlo + up(nk * I);
  L.obuf = L.hsc + up(nk * kb4_of(I));
  L.total = L.obuf + up(2 * nk * H);
  return L;
}

}  // namespace

hipError_t launch_mfma_probe(bool f8f4, int blocks, int iters, float *sink, hipStream_t s) {
  if (f8f4) hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, iters, sink, 127);
  else hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, iters, sink, 127);
  return hipGetLastError();
}

int64_t mfma_probe_flops(bool f8f4, int blocks, int iters) {
  return (int64_t)blocks * (kThreads / 64) * iters * kProbeChains * 32 * 32 * (f8f4 ? 64 : 16) * 2;
}

bool prefill_supported(int H, int I, int E) {
  return H % 64 == 0 && I % 64 == 0 && H / 32 <= kMaxKb && I / 32 <= kMaxKb && E <= OES_MAX_EXPERTS;
}

int64_t prefill_workspace_bytes(int H, int I, int n, int k, int E) { return ws_layout(H, I, n, k, E).total; }

hipError_t launch_prefill_ffn(const PrefillArgs &a, hipStream_t s) {
  if (!prefill_supported(a.H, a.I, a.E)) return hipErrorInvalidValue;
  // A byte offsets of the GEMMs (row * K) are 32-bit
  if ((int64_t)a.n * a.k * std::max(a.H, a.I) >= (int64_t)1 << 31) return hipErrorInvalidValue;
  const WsLayout L = ws_layout(a.H, a.I, a.n, a.k, a.E);
  if (a.ws_bytes < L.total) return hipErrorInvalidValue;
  const int nk = a.n * a.k;
  int32_t *offsets = reinterpret_cast<int32_t *>(a.ws + L.offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(a.ws + L.perm);
  int32_t *order = reinterpret_cast<int32_t *>(a.ws + L.order);
  int32_t *pos = reinterpret_cast<int32_t *>(a.ws + L.pos);
  uint32_t *zeros = reinterpret_cast<uint32_t *>(a.ws + L.zeros);
  PrepArgs pa;
  pa.ids = a.ids;
  pa.nk = nk;
  pa.E = a.E;
  pa.offsets = offsets;
  pa.perm = perm;
  pa.pos = pos;
  pa.order = order;
  pa.zeros = zeros;
  pa.x = a.x;
  pa.count = (int64_t)a.n * a.H;
  pa.K = a.H;
  pa.hi = a.ws + L.xhi;
  pa.lo = a.ws + L.xlo;
  pa.sc = a.ws + L.xsc;
  const int64_t split_blocks = (pa.count / 8 + kPrepThreads - 1) / kPrepThreads;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(1 + split_blocks)), dim3(kPrepThreads), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemmArgs g;
  g.zero16 = reinterpret_cast<const u32x4 *>(zeros);
  g.H = a.H;
  g.I = a.I;
  g.E = a.E;
  g.k = a.k;
  g.nk = nk;
  g.xcd = (a.E % kXcds == 0) ? 1 : 0;
  g.offsets = offsets;
  g.perm = perm;
  g.order = order;
  g.hhi = a.ws + L.hhi;
  g.hlo = a.ws + L.hlo;
  g.hsc = a.ws + L.hsc;
  g.obuf = reinterpret_cast<uint16_t *>(a.ws + L.obuf);
  // gate_up: banks 0..2, A = the split x; features I, 128 per block
  g.ahi = a.ws + L.xhi;
  g.alo = a.ws + L.xlo;
  g.asc = a.ws + L.xsc;
  g.blocks = a.bank[0];
  g.scales = a.bank[1];
  g.bias = reinterpret_cast<const uint16_t *>(a.bank[2]);
  g.blocks_stride = a.row_bytes[0];
  g.scales_stride = a.row_bytes[1];
  g.bias_stride = a.row_bytes[2] / 2;
  g.ntiles = (a.I + 127) / 128;
  hipLaunchKernelGGL(moe_gemm_kernel<0>, dim3(a.E * g.ntiles), dim3(kThreads), 0, s, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // down: banks 3..5, A = the split h; features H, 256 per block
  g.ahi = g.hhi;
  g.alo = g.hlo;
  g.asc = g.hsc;
  g.blocks = a.bank[3];
  g.scales = a.bank[4];
  g.bias = reinterpret_cast<const uint16_t *>(a.bank[5]);
  g.blocks_stride = a.row_bytes[3];
  g.scales_stride = a.row_bytes[4];
  g.bias_stride = a.row_bytes[5] / 2;
  g.ntiles = (a.H + 255) / 256;
  hipLaunchKernelGGL(moe_gemm_kernel<1>, dim3(a.E * g.ntiles), dim3(kThreads), 0, s, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid((a.H / 4 + kThreads - 1) / kThreads, a.n);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(kThreads), 0, s, g.obuf, pos, a.ids, a.w, a.n, a.k, a.H, a.E, a.y);
  return hipGetLastError();
}

}  // namespace oes
