"""Pins of the oracle expert FFN and its dequantisation.

* bf16 (exact decode): the oracle equals a dense SwiGLU MLP computed by an
  independent expression (torch float64 linear/silu) for a single token and a
  single expert with weight 1, and a weighted sum over several experts.
* Quantised formats: the dequantised weights equal the float32 draws the
  generator encoded, within the format's rounding error (a swapped nibble,
  transposed block or dropped scale fails this by orders of magnitude); fp8
  block dequant also equals torch's own e4m3 conversion times the expanded
  scale.
* x = 0 gives the closed form sum_j w_j (b_d + Wd (silu(b_g) * b_u)).
* Permuting slots, and linearity in the routing weights.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import synth
from oracle import ffn, schema


def _rows_np(rows):
    return [r.numpy().copy() for r in rows]


def _x_bits(n, H, seed=0):
    return synth.activations(n, H, seed, "ffn-test").numpy().view(np.uint16)


def test_bf16_single_expert_equals_dense_swiglu():
    H, I = 64, 48
    rows = synth.expert_rows("bf16", H, I, 0, "t", 3)
    xb = _x_bits(1, H)
    y = ffn.expert_ffn("bf16", H, I, xb, np.array([[0]]), np.array([[1.0]]), lambda s: _rows_np(rows))
    wgu = rows[0].view(torch.bfloat16).reshape(2 * I, H).double()
    wd = rows[1].view(torch.bfloat16).reshape(H, I).double()
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double()
    ref = Fn.linear(Fn.silu(Fn.linear(x, wgu[:I])) * Fn.linear(x, wgu[I:]), wd)
    assert ffn.rel_l2(y, ref.numpy()) < 1e-12


def test_bf16_weighted_combine_equals_dense():
    H, I, k = 32, 16, 3
    experts = [synth.expert_rows("bf16", H, I, 0, "t", e) for e in range(k)]
    xb = _x_bits(2, H, 1)
    w = np.array([[0.5, 0.3, 0.2], [0.1, 0.1, 0.8]])
    slot_ids = np.array([[0, 1, 2], [2, 0, 1]])
    y = ffn.expert_ffn("bf16", H, I, xb, slot_ids, w, lambda s: _rows_np(experts[s]))
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double()
    ref = torch.zeros(2, H, dtype=torch.float64)
    for t in range(2):
        for j in range(k):
            r = experts[slot_ids[t, j]]
            wgu = r[0].view(torch.bfloat16).reshape(2 * I, H).double()
            wd = r[1].view(torch.bfloat16).reshape(H, I).double()
            a = wgu @ x[t]
            ref[t] += w[t, j] * (wd @ (Fn.silu(a[:I]) * a[I:]))
    assert ffn.rel_l2(y, ref.numpy()) < 1e-12


@pytest.mark.parametrize("fmt,H,I,bound", [
    ("bf16", 256, 128, 0.004),
    ("fp8_block128", 256, 128, 0.05),
    ("nvfp4", 64, 32, 0.15),
    ("mxfp4_t", 64, 64, 0.2),
    ("q4_0", 256, 128, 0.15),
])
def test_dequant_round_trip(fmt, H, I, bound):
    wgu, wd, bgu, bd = synth.expert_weights(fmt, H, I, 0, "rt", 11)
    rows = synth.encode_expert(fmt, wgu, wd, bgu, bd)
    dg, dd, dbg, dbd = ffn.dequant_expert(fmt, H, I, _rows_np(rows))
    for got, ref in ((dg, wgu), (dd, wd)):
        ref = ref.double().numpy()
        err = ffn.rel_l2(got, ref)
        assert err < bound, (fmt, err)
        # a transposed or swapped decode is far off
        assert ffn.rel_l2(got.T.reshape(ref.shape) if got.shape[0] != got.shape[1] else got.T, ref) > 0.5
    if fmt == "mxfp4_t":
        assert ffn.rel_l2(dbg, bgu.double().numpy()) < 0.004
        assert ffn.rel_l2(dbd, bd.double().numpy()) < 0.004


def test_fp8_dequant_equals_library_conversion():
    H, I = 256, 128
    rows = synth.expert_rows("fp8_block128", H, I, 0, "lib", 2)
    dg, dd, _, _ = ffn.dequant_expert("fp8_block128", H, I, _rows_np(rows))
    q = rows[0].view(torch.float8_e4m3fn).reshape(2 * I, H).double()
    s = rows[1].view(torch.float32).reshape(2 * I // 128, H // 128).double()
    ref = q * s.repeat_interleave(128, 0).repeat_interleave(128, 1)
    assert np.array_equal(dg, ref.numpy())


def test_nvfp4_dequant_structure():
    # codes that all decode to +1 with scale byte 0x38 (e4m3 1.0) and global fp16 1.0 -> all ones
    H, I = 32, 16
    specs = schema.bank_specs("nvfp4", H, I)
    rows = []
    for name, elem, shape, nbytes in specs:
        if name.endswith("codes"):
            rows.append(np.full(nbytes, 0x22, dtype=np.uint8))       # two codes of value 1.0
        elif name.endswith("scale"):
            rows.append(np.full(nbytes, 0x38, dtype=np.uint8))
        else:
            rows.append(np.frombuffer(np.full(nbytes // 2, 1.0, dtype=np.float16).tobytes(), dtype=np.uint8))
    dg, dd, _, _ = ffn.dequant_expert("nvfp4", H, I, rows)
    assert (dg == 1.0).all() and (dd == 1.0).all()


def test_q4_0_dequant_structure():
    # codes 0x99 (q = 9 -> +1) with d = fp16 0.25 -> every weight 0.25; codes 0x88 -> 0
    H, I = 64, 32
    for byte, want in ((0x99, 0.25), (0x88, 0.0), (0x70, None)):
        rows = []
        for name, elem, shape, nbytes in schema.bank_specs("q4_0", H, I):
            if name.endswith("_q"):
                rows.append(np.full(nbytes, byte, dtype=np.uint8))
            else:
                rows.append(np.frombuffer(np.full(nbytes // 2, 0.25, dtype=np.float16).tobytes(), dtype=np.uint8))
        dg, dd, _, _ = ffn.dequant_expert("q4_0", H, I, rows)
        if want is not None:
            assert (dg == want).all() and (dd == want).all()
        else:
            # 0x70: low nibble 0 -> -8 * 0.25 for the first 16 of every 32, high nibble 7 -> -0.25
            blk = dg.reshape(2 * I, H // 32, 32)
            assert (blk[:, :, :16] == -2.0).all() and (blk[:, :, 16:] == -0.25).all()


@pytest.mark.parametrize("fmt,H,I", [("bf16", 32, 16), ("mxfp4_t", 64, 32)])
def test_zero_input_closed_form(fmt, H, I):
    """x = 0: y = sum_j w_j (b_d + Wd (silu(b_gate) * b_up)), which is 0 without biases.
    The MXFP4 side is evaluated from a decoder written apart from the oracle (literal
    OCP e2m1 table, torch's e8m0 type, torch's SiLU), in torch float64."""
    import torch

    from tests import mxfp4_torch_ref as ref
    experts = [synth.expert_rows(fmt, H, I, 0, "z", e) for e in range(2)]
    w = np.array([[0.7, 0.3]])
    xb = np.zeros((1, H), dtype=np.uint16)
    y = ffn.expert_ffn(fmt, H, I, xb, np.array([[0, 1]]), w, lambda s: _rows_np(experts[s]))
    if fmt == "bf16":
        assert (y == 0).all()
        return
    want = torch.zeros(H, dtype=torch.float64)
    for j in range(2):
        _, wd, bgu, bd = ref.expert(_rows_np(experts[j]), H, I)
        want += w[0, j] * (bd + wd @ (torch.nn.functional.silu(bgu[:I]) * bgu[I:]))
    assert np.allclose(y[0], want.numpy(), rtol=1e-12, atol=0)
    assert want.abs().max() > 0


def test_mxfp4_decoder_matches_independent_torch_decoder():
    """The oracle's MXFP4 (transposed) dequant against the torch-float64 decoder on
    seeded experts and on bytes covering every code and a spread of scales."""
    from tests import mxfp4_torch_ref as ref
    H, I = 64, 32
    rows = _rows_np(synth.expert_rows("mxfp4_t", H, I, 0, "dq", 5))
    wgu, wd, bgu, bd = ffn.dequant_expert("mxfp4_t", H, I, rows)
    tg, td, tbg, tbd = ref.expert(rows, H, I)
    assert np.array_equal(wgu, tg.numpy()) and np.array_equal(wd, td.numpy())
    assert np.array_equal(bgu, tbg.numpy()) and np.array_equal(bd, tbd.numpy())
    rng = np.random.default_rng(3)
    raw = [r.copy() for r in rows]
    raw[0] = rng.integers(0, 256, raw[0].size, dtype=np.uint8)         # every code
    raw[1] = rng.integers(100, 155, raw[1].size, dtype=np.uint8)       # scales 2^-27 .. 2^27
    raw[3] = rng.integers(0, 256, raw[3].size, dtype=np.uint8)
    raw[4] = rng.integers(100, 155, raw[4].size, dtype=np.uint8)
    wgu, wd, _, _ = ffn.dequant_expert("mxfp4_t", H, I, raw)
    tg, td, _, _ = ref.expert(raw, H, I)
    assert np.array_equal(wgu, tg.numpy()) and np.array_equal(wd, td.numpy())


def test_slot_permutation_and_linearity():
    H, I = 32, 16
    experts = [synth.expert_rows("bf16", H, I, 0, "p", e) for e in range(4)]
    xb = _x_bits(3, H, 2)
    ids = np.array([[0, 3], [1, 2], [3, 3]])
    w = np.array([[0.6, 0.4], [0.5, 0.5], [0.9, 0.1]])
    y = ffn.expert_ffn("bf16", H, I, xb, ids, w, lambda s: _rows_np(experts[s]))
    perm = [2, 0, 3, 1]                    # expert e lives in slot perm[e]
    inv = {perm[e]: e for e in range(4)}
    y2 = ffn.expert_ffn("bf16", H, I, xb, np.vectorize(lambda e: perm[e])(ids), w,
                        lambda s: _rows_np(experts[inv[s]]))
    assert np.allclose(y, y2, rtol=1e-13, atol=1e-15)
    y3 = ffn.expert_ffn("bf16", H, I, xb, ids, 2.5 * w, lambda s: _rows_np(experts[s]))
    assert np.allclose(y3, 2.5 * y, rtol=1e-13)
    skip = ids.copy()
    skip[0, 1] = -1
    y4 = ffn.expert_ffn("bf16", H, I, xb, skip, w, lambda s: _rows_np(experts[s]))
    w0 = w.copy()
    w0[0, 1] = 0.0
    y5 = ffn.expert_ffn("bf16", H, I, xb, ids, w0, lambda s: _rows_np(experts[s]))
    assert np.allclose(y4, y5, rtol=1e-13, atol=1e-15)
