"""Seeded synthetic inputs for the offloaded-expert step (shared by tests, bench and smoke).

This module produces input bytes only: expert weights drawn from a normal
distribution and encoded into each bank format, activations, router weights,
router logits, synthetic routed ids and the initial slot-table state of the copy
benchmark.  It holds none of the step's arithmetic (no routing, no LRU, no
copy, no decoding, no FFN): the encoders below turn float32 draws into the
bytes a bank stores, the inverse of what the step reads.

Streams: every tensor is drawn from its own generator seeded by a 63-bit key
hashed from (seed, labels...), so any single expert's rows can be regenerated
alone.  Draws use torch's generator on the requested device; the CPU and GPU
generators give different (each deterministic) values, which is fine because
every check reads back the very bytes that were generated.

Encoders (public format recipes, not from the pages):
  bf16        round to nearest even (torch conversion)
  fp8 block   per 128x128 block s = max(amax, tiny) / 448, q = e4m3(clip(w / s, +-448))
  nvfp4       per row g = fp16(max(amax_row, tiny) / (6 * 448)); per 16 along K
              sc = e4m3(amax_blk / (6 g)) clamped to [2**-9, 448];
              q = e2m1(clip(w / (sc g), +-6)); two codes per byte, low nibble first
  mxfp4 (T)   per 32 along K, exponent e = clip(floor(log2 amax) - 2 + 127, 0, 254),
              q = e2m1(clip(w / 2**(e - 127), +-6)); blocks laid out [K/32, N, 16]
  q4_0        per 32 along K d = fp16(max(amax, tiny) / 7), q = clip(round(w / d) + 8, 0, 15);
              byte j of a block holds q_j | q_(j+16) << 4 (GGUF block_q4_0 order)
e2m1 rounding is to nearest, ties to the even code.
"""
import hashlib

import numpy as np
import torch

FORMATS = ("bf16", "fp8_block128", "nvfp4", "mxfp4_t", "q4_0")
WEIGHT_STD = 0.02


# ----------------------------------------------------------------------------- streams
def stream_key(*labels) -> int:
    h = hashlib.blake2b(repr(labels).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def normal(shape, key, std=1.0, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(key))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def _u8(t):
    return t.contiguous().view(torch.uint8).reshape(-1)


# ----------------------------------------------------------------------------- encoders
def bf16_bits(t):
    """float32 tensor -> bf16 bit patterns as an int16 tensor (round to nearest even)."""
    return t.to(torch.bfloat16).view(torch.int16)


def _e2m1_codes(v):
    """Values already clipped to [-6, 6] -> 4-bit e2m1 codes (uint8), ties to even code."""
    a = v.abs()
    mids = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
    code = torch.zeros_like(a, dtype=torch.uint8)
    for i, m in enumerate(mids):
        code += ((a > m) if i % 2 == 0 else (a >= m)).to(torch.uint8)
    neg = (v < 0) & (code > 0)
    return code | (neg.to(torch.uint8) << 3)


def _pack_low_first(codes):
    """[..., 2m] codes -> [..., m] bytes, element 2j in the low nibble."""
    return codes[..., 0::2] | (codes[..., 1::2] << 4)


def fp8_block_encode(w):
    """[R, C] float32 (R, C multiples of 128) -> (q uint8 [R, C], scale float32 [R/128, C/128])."""
    R, C = w.shape
    blk = w.reshape(R // 128, 128, C // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = torch.clamp(amax, min=1e-12) / 448.0
    q = (blk / s[:, None, :, None]).clamp(-448.0, 448.0).reshape(R, C).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s.to(torch.float32)


def nvfp4_encode(w):
    """[R, K] float32 -> (codes uint8 [R, K/2], scale e4m3 uint8 [R, K/16], global fp16 bits int16 [R])."""
    R, K = w.shape
    g = (torch.clamp(w.abs().amax(dim=1), min=1e-12) / (6.0 * 448.0)).to(torch.float16)
    g32 = g.to(torch.float32)
    blk = w.reshape(R, K // 16, 16)
    amax = blk.abs().amax(dim=2)
    sc = (amax / (6.0 * g32[:, None])).clamp(2.0 ** -9, 448.0).to(torch.float8_e4m3fn)
    sc32 = sc.to(torch.float32)
    q = (blk / (sc32[:, :, None] * g32[:, None, None])).clamp(-6.0, 6.0).reshape(R, K)
    codes = _pack_low_first(_e2m1_codes(q))
    return codes, sc.view(torch.uint8), g.view(torch.int16)


def mxfp4_t_encode(w):
    """[N, K] float32 -> (blocks uint8 [K/32, N, 16], scales e8m0 uint8 [K/32, N])."""
    N, K = w.shape
    blk = w.reshape(N, K // 32, 32)
    amax = blk.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                 # amax = m * 2**ex, m in [0.5, 1)
    e = torch.where(amax > 0, ex - 1 - 2 + 127, torch.zeros_like(ex)).clamp(0, 254)
    scale = torch.pow(2.0, (e - 127).to(torch.float32))
    q = (blk / scale[:, :, None]).clamp(-6.0, 6.0)
    codes = _pack_low_first(_e2m1_codes(q))   # [N, K/32, 16]
    return codes.permute(1, 0, 2).contiguous(), e.to(torch.uint8).t().contiguous()


def q4_0_encode(w):
    """[R, K] float32 (K % 32 == 0) -> (codes uint8 [R, K/2] in GGUF block order, d fp16 bits int16 [R, K/32]).

    d = amax / 7 of each 32-block (fp16), q = clip(round(w / d) + 8, 0, 15);
    byte j of a block holds q[j] (low nibble) and q[j + 16] (high nibble).
    """
    R, K = w.shape
    blk = w.reshape(R, K // 32, 32)
    d = (torch.clamp(blk.abs().amax(dim=2), min=1e-6) / 7.0).to(torch.float16)
    q = (torch.round(blk / d.to(torch.float32)[:, :, None]) + 8).clamp(0, 15).to(torch.uint8)
    codes = q[..., :16] | (q[..., 16:] << 4)
    return codes.reshape(R, K // 2), d.view(torch.int16)


# ----------------------------------------------------------------------------- experts
def expert_weights(fmt, hidden, inter, seed, tag, flat_id, device="cpu"):
    """float32 draws (Wgu [2I, H], Wd [H, I], b_gu [2I] or None, b_d [H] or None) of one expert."""
    wgu = normal((2 * inter, hidden), stream_key(seed, tag, "gate_up", flat_id), WEIGHT_STD, device)
    wd = normal((hidden, inter), stream_key(seed, tag, "down", flat_id), WEIGHT_STD, device)
    bgu = bd = None
    if fmt == "mxfp4_t":
        bgu = normal((2 * inter,), stream_key(seed, tag, "gate_up_bias", flat_id), WEIGHT_STD, device)
        bd = normal((hidden,), stream_key(seed, tag, "down_bias", flat_id), WEIGHT_STD, device)
    return wgu, wd, bgu, bd


def encode_expert(fmt, wgu, wd, bgu=None, bd=None):
    """Encode one expert's float32 weights into its bank rows (list of flat uint8 tensors, bank order)."""
    if fmt == "bf16":
        return [_u8(bf16_bits(wgu)), _u8(bf16_bits(wd))]
    if fmt == "fp8_block128":
        q1, s1 = fp8_block_encode(wgu)
        q2, s2 = fp8_block_encode(wd)
        return [_u8(q1), _u8(s1), _u8(q2), _u8(s2)]
    if fmt == "nvfp4":
        c1, s1, g1 = nvfp4_encode(wgu)
        c2, s2, g2 = nvfp4_encode(wd)
        return [_u8(c1), _u8(s1), _u8(g1), _u8(c2), _u8(s2), _u8(g2)]
    if fmt == "q4_0":
        q1, d1 = q4_0_encode(wgu)
        q2, d2 = q4_0_encode(wd)
        return [_u8(q1), _u8(d1), _u8(q2), _u8(d2)]
    if fmt == "mxfp4_t":
        b1, s1 = mxfp4_t_encode(wgu)
        b2, s2 = mxfp4_t_encode(wd)
        return [_u8(b1), _u8(s1), _u8(bf16_bits(bgu)), _u8(b2), _u8(s2), _u8(bf16_bits(bd))]
    raise ValueError(fmt)


def expert_rows(fmt, hidden, inter, seed, tag, flat_id, device="cpu"):
    """Bank rows of one expert, drawn from its own streams and encoded."""
    return encode_expert(fmt, *expert_weights(fmt, hidden, inter, seed, tag, flat_id, device))


def fill_layer_banks(fmt, hidden, inter, num_experts, layer, seed, tag, banks, device="cpu"):
    """Write every expert of `layer` into host bank tensors.

    banks[b] is a uint8 tensor of E * row_bytes_b bytes (e.g. pinned host memory).
    Rows are generated on `device` and copied in.
    """
    for e in range(num_experts):
        fid = layer * num_experts + e
        rows = expert_rows(fmt, hidden, inter, seed, tag, fid, device)
        for b, r in enumerate(rows):
            nb = r.numel()
            banks[b][e * nb:(e + 1) * nb].copy_(r, non_blocking=False)


# ----------------------------------------------------------------------------- activations
def activations(n, hidden, seed, tag, step=0, device="cpu"):
    """x[n, H] ~ N(0, 1) as bf16 bit patterns (int16)."""
    return bf16_bits(normal((n, hidden), stream_key(seed, tag, "x", step), 1.0, device))


def router_weight(hidden, num_experts, seed, tag, device="cpu"):
    """Wg[H, E] ~ N(0, 0.02) as bf16 bit patterns (int16)."""
    return bf16_bits(normal((hidden, num_experts), stream_key(seed, tag, "wg"), WEIGHT_STD, device))


def router_logits(n, num_experts, seed, tag, device="cpu"):
    """Router logits [n, E] ~ N(0, 1), float32 (the prefill workload routes given logits)."""
    return normal((n, num_experts), stream_key(seed, tag, "logits"), 1.0, device)


# ----------------------------------------------------------------------------- copy-benchmark setup
def synthetic_ids(n, k, num_experts, seed, tag):
    """Routed ids whose distinct count is exactly min(E, n*k).

    ids[t, j] = perm[(t*k + j) mod E] for a seeded permutation of the experts.
    """
    g = torch.Generator().manual_seed(stream_key(seed, tag, "perm", n, k))
    perm = torch.randperm(num_experts, generator=g)
    idx = torch.arange(n * k) % num_experts
    return perm[idx].reshape(n, k).to(torch.int32)


def foreign_state(num_slots, num_experts):
    """Initial slot table with every slot owned by another layer's expert.

    owner[s] = E + s (layer >= 1), stamps 0, clock 0; with layer 0 driven this
    layer never hits, and victims are taken in slot order.
    """
    owner = np.arange(num_slots, dtype=np.int64) + num_experts
    stamp = np.zeros(num_slots, dtype=np.uint64)
    return owner, stamp, 0


def forced_miss_state(num_slots, num_experts, layer, ids, misses):
    """Slot table that makes exactly `misses` of the step's distinct ids miss.

    Distinct requested flat ids U (ascending): the last `misses` of them miss;
    the others are pre-installed into the highest-index slots (their rows must
    then be loaded into those slots).  Every other slot keeps a foreign owner.
    Returns (owner, stamp, clock, preinstalled [(slot, flat_id)]).
    """
    owner, stamp, clock = foreign_state(num_slots, num_experts)
    U = sorted(set(int(layer * num_experts + int(e)) for e in np.asarray(ids).ravel()))
    if not 0 <= misses <= len(U):
        raise ValueError("misses out of range")
    hits = U[:len(U) - misses]
    if len(hits) > num_slots:
        raise ValueError("more hits than slots")
    pre = []
    for i, fid in enumerate(hits):
        s = num_slots - 1 - i
        owner[s] = fid
        pre.append((s, fid))
    return owner, stamp, clock, pre
