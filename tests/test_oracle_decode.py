"""Pins of the oracle's bit-field decoders against library conversions and the OCP tables."""
import os

import numpy as np
import torch

from oracle import decode


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    nan_a, nan_b = np.isnan(a), np.isnan(b)
    assert (nan_a == nan_b).all()
    ok = ~nan_a
    assert np.array_equal(a[ok], b[ok])
    # signed zeros must match too
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


def test_bf16_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    _same(decode.bf16(bits), ref)


def test_fp16_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    _same(decode.fp16(bits), bits.view(np.float16).astype(np.float64))


def test_e4m3_all_codes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _same(decode.e4m3(b), ref)
    assert decode.e4m3(np.uint8(0x7E)) == 448.0


def test_e8m0_all_codes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    _same(decode.e8m0(b), ref)
    assert decode.e8m0(np.uint8(127)) == 1.0


def test_e2m1_table():
    # OCP Microscaling v1.0, FP4 E2M1 element values
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    want = table + [-v for v in table]
    got = decode.e2m1(np.arange(16))
    _same(got, want)


def test_e2m1_matches_torch_if_available():
    try:
        packed = torch.arange(256, dtype=torch.uint8).view(torch.float4_e2m1fn_x2)
        vals = packed.to(torch.float32)  # may not be supported
    except Exception:
        return
    # torch's unpack order is not documented; check the value multiset only
    got = np.sort(decode.e2m1(decode.fp4x2_unpack(np.arange(256, dtype=np.uint8)[:, None]).ravel()))
    assert np.array_equal(np.sort(vals.double().numpy().ravel()), got)


def test_fp4x2_unpack_order():
    # reading: element 2j in the low nibble of byte j
    codes = decode.fp4x2_unpack(np.array([[0x21, 0xF7]], dtype=np.uint8))
    assert codes.tolist() == [[1, 2, 7, 15]]


def test_table_evaluation_equals_direct():
    rng = np.random.default_rng(4)
    b = rng.integers(0, 256, size=(7, 33), dtype=np.uint8)
    for fn, n in ((decode.e4m3, 256), (decode.e8m0, 256)):
        _same(decode.via_table(fn, b, n), fn(b))
    c = rng.integers(0, 16, size=(5, 9))
    _same(decode.via_table(decode.e2m1, c, 16), decode.e2m1(c))


def test_q4_0_golden_block():
    """A GGUF Q4_0 block worked by hand (tests/golden/q4_0_block.txt)."""
    lines = [l.split("#")[0].split() for l in open(os.path.join(os.path.dirname(__file__), "golden", "q4_0_block.txt"))]
    kv = {l[0]: l[1:] for l in lines if l}
    d = decode.fp16(np.array([int(kv["d_bits"][0], 16)], dtype=np.uint16))[0]
    codes = np.array([int(b, 16) for b in kv["bytes"]], dtype=np.uint8)
    got = decode.q4_0(decode.q4x2_unpack(codes)) * d
    assert got.tolist() == [float(v) for v in kv["values"]]


def test_q4x2_unpack_blocks_are_independent():
    rng = np.random.default_rng(3)
    a = rng.integers(0, 256, size=(5, 64), dtype=np.uint8)          # 4 blocks per row
    whole = decode.q4x2_unpack(a)
    for b in range(4):
        assert np.array_equal(whole[:, 32 * b:32 * b + 32], decode.q4x2_unpack(a[:, 16 * b:16 * b + 16]))
    # element j + 16 of a block is the high nibble of byte j, not of byte 2j or 2j+1
    assert np.array_equal(whole[:, 16:32], a[:, :16] >> 4)
