"""The grouped SwiGLU expert FFN computed on the slot cache, with top-k weighted combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FreeToken architecture walk-through §5 and FreeToken MoE benchmark guide §1
(background) and §4.2: hits are computed straight from the slot cache; the
banks hold the expert FFN weights in one of the quantised formats.  For every
token t and routed expert j (weight w[t, j], slot s = slot_ids[t, j]):

    a   = Wgu[s] . x_t (+ gate_up bias)        a has 2I entries
    g   = a[:I], u = a[I:]
    h   = silu(g) * u,   silu(g) = g / (1 + exp(-g))
    o   = Wd[s] . h   (+ down bias)            o has H entries
    y_t = sum_j w[t, j] * o

Dequantisation (readings; formats from the pages' bank list):
  bf16        W = bf16(bits)
  fp8 block   W[r, c] = e4m3(q[r, c]) * scale[r // 128, c // 128]
  nvfp4       W[r, c] = e2m1(code[r, c]) * e4m3(scale[r, c // 16]) * fp16(global[r])
  mxfp4 (T)   W[n, c] = e2m1(code of blocks[c // 32, n, (c % 32) // 2], nibble c % 2)
                        * 2 ** (scales[c // 32, n] - 127), plus a bf16 bias per output
  q4_0        W[r, c] = (q[r, c] - 8) * fp16(d[r, c // 32]), q unpacked in GGUF block order

Everything is float64.  A slot id of -1 contributes nothing (reserved for
experts computed elsewhere).
"""
import numpy as np

from . import decode, schema


def _rows(bank_rows, name, specs):
    for (nm, elem, shape, nbytes), raw in zip(specs, bank_rows):
        if nm == name:
            raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
            if raw.size != nbytes:
                raise ValueError(f"bank {name}: {raw.size} bytes, expected {nbytes}")
            return elem, shape, raw
    raise KeyError(name)


def _bf16_matrix(raw, shape):
    return decode.bf16(raw.view(np.uint16).reshape(shape))


def _fp8_matrix(raw_q, shape, raw_s, sshape):
    q = decode.via_table(decode.e4m3, raw_q.reshape(shape), 256)
    s = raw_s.view(np.float32).reshape(sshape).astype(np.float64)
    return q * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)


def _nvfp4_matrix(raw_c, cshape, raw_s, sshape, raw_g):
    rows, half = cshape
    codes = decode.fp4x2_unpack(raw_c.reshape(rows, half))          # [rows, K]
    vals = decode.via_table(decode.e2m1, codes, 16)
    sc = decode.via_table(decode.e4m3, raw_s.reshape(sshape), 256)   # [rows, K/16]
    g = decode.fp16(raw_g.view(np.uint16))                           # [rows]
    return vals * np.repeat(sc, 16, axis=1) * g[:, None]


def _mxfp4_matrix(raw_b, bshape, raw_s, sshape):
    kb, n, _ = bshape
    blocks = raw_b.reshape(bshape)                                   # [K/32, N, 16]
    codes = decode.fp4x2_unpack(blocks)                              # [K/32, N, 32]
    vals = decode.via_table(decode.e2m1, codes, 16) * decode.e8m0(raw_s.reshape(sshape))[:, :, None]
    # W[n, c] with c = 32 * kb + position in block
    return vals.transpose(1, 0, 2).reshape(n, kb * 32)


def _q4_0_matrix(raw_q, qshape, raw_d, dshape):
    rows, half = qshape
    vals = decode.q4_0(decode.q4x2_unpack(raw_q.reshape(rows, half)))   # [rows, K]
    d = decode.fp16(raw_d.view(np.uint16).reshape(dshape))               # [rows, K/32]
    return vals * np.repeat(d, 32, axis=1)


def dequant_expert(fmt, hidden, inter, bank_rows):
    """One expert's rows (one uint8 array per bank, schema order) -> (Wgu, Wd, b_gu, b_d) in float64."""
    specs = schema.bank_specs(fmt, hidden, inter)
    if len(bank_rows) != len(specs):
        raise ValueError("wrong number of banks")
    bgu = bd = None
    if fmt == schema.BF16:
        _, s1, r1 = _rows(bank_rows, "gate_up", specs)
        _, s2, r2 = _rows(bank_rows, "down", specs)
        wgu, wd = _bf16_matrix(r1, s1), _bf16_matrix(r2, s2)
    elif fmt == schema.FP8_BLOCK128:
        _, s1, r1 = _rows(bank_rows, "gate_up", specs)
        _, ss1, rs1 = _rows(bank_rows, "gate_up_scale", specs)
        _, s2, r2 = _rows(bank_rows, "down", specs)
        _, ss2, rs2 = _rows(bank_rows, "down_scale", specs)
        wgu, wd = _fp8_matrix(r1, s1, rs1, ss1), _fp8_matrix(r2, s2, rs2, ss2)
    elif fmt == schema.NVFP4:
        _, c1, rc1 = _rows(bank_rows, "gate_up_codes", specs)
        _, ss1, rs1 = _rows(bank_rows, "gate_up_scale", specs)
        _, _, rg1 = _rows(bank_rows, "gate_up_global", specs)
        _, c2, rc2 = _rows(bank_rows, "down_codes", specs)
        _, ss2, rs2 = _rows(bank_rows, "down_scale", specs)
        _, _, rg2 = _rows(bank_rows, "down_global", specs)
        wgu = _nvfp4_matrix(rc1, c1, rs1, ss1, rg1)
        wd = _nvfp4_matrix(rc2, c2, rs2, ss2, rg2)
    elif fmt == schema.MXFP4_T:
        _, b1, rb1 = _rows(bank_rows, "gate_up_blocks", specs)
        _, ss1, rs1 = _rows(bank_rows, "gate_up_scales", specs)
        _, _, rbias1 = _rows(bank_rows, "gate_up_bias", specs)
        _, b2, rb2 = _rows(bank_rows, "down_blocks", specs)
        _, ss2, rs2 = _rows(bank_rows, "down_scales", specs)
        _, _, rbias2 = _rows(bank_rows, "down_bias", specs)
        wgu, wd = _mxfp4_matrix(rb1, b1, rs1, ss1), _mxfp4_matrix(rb2, b2, rs2, ss2)
        bgu = decode.bf16(rbias1.view(np.uint16))
        bd = decode.bf16(rbias2.view(np.uint16))
    elif fmt == schema.Q4_0:
        _, q1, rq1 = _rows(bank_rows, "gate_up_q", specs)
        _, d1, rd1 = _rows(bank_rows, "gate_up_d", specs)
        _, q2, rq2 = _rows(bank_rows, "down_q", specs)
        _, d2, rd2 = _rows(bank_rows, "down_d", specs)
        wgu, wd = _q4_0_matrix(rq1, q1, rd1, d1), _q4_0_matrix(rq2, q2, rd2, d2)
    else:
        raise ValueError(fmt)
    if wgu.shape != (2 * inter, hidden) or wd.shape != (hidden, inter):
        raise AssertionError("dequantised shapes disagree with the schema")
    return wgu, wd, bgu, bd


def silu(g):
    return g / (1.0 + np.exp(-g))


def expert_out(x64, wgu, wd, bgu=None, bd=None):
    """o = Wd . (silu(gate) * up) (+ biases), float64.

    x64 is [H] for one token or [m, H] for m tokens routed to the same expert
    (then o is [m, H]); the matrix form is the same formula applied row by row.
    """
    inter = wd.shape[1]
    a = x64 @ wgu.T
    if bgu is not None:
        a = a + bgu
    h = silu(a[..., :inter]) * a[..., inter:]
    o = h @ wd.T
    if bd is not None:
        o = o + bd
    return o


def expert_ffn(fmt, hidden, inter, x_bits, slot_ids, w, slot_row_fn):
    """y[n, H] (float64) of the routed tokens.

    x_bits      - uint16 bf16 bits [n, H]
    slot_ids    - int [n, k]; -1 skips the pair
    w           - routing weights [n, k]
    slot_row_fn - slot_row_fn(slot) -> list of this slot's rows (uint8, schema order)

    Experts are dequantised one distinct slot at a time; every (t, j) pair
    routed to that slot adds w[t, j] * o to y[t].
    """
    x = decode.bf16(np.asarray(x_bits, dtype=np.uint16))
    slot_ids = np.asarray(slot_ids)
    w = np.asarray(w, dtype=np.float64)
    n, k = slot_ids.shape
    y = np.zeros((n, hidden), dtype=np.float64)
    for s in sorted(set(int(v) for v in slot_ids.ravel() if v >= 0)):
        tt, jj = np.nonzero(slot_ids == s)
        wgu, wd, bgu, bd = dequant_expert(fmt, hidden, inter, slot_row_fn(s))
        o = expert_out(x[tt], wgu, wd, bgu, bd)
        np.add.at(y, tt, w[tt, jj][:, None] * o)
    return y


def rel_l2(y, y_ref):
    """||y - y_ref||_2 / ||y_ref||_2 over the whole output."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))
