"""The arithmetic behind the prefill GEMM's activation planes, checked on the CPU.

The grouped GEMM feeds each bf16 activation to an e4m3 x e2m1 block-scaled MFMA
as two e4m3 codes: with s chosen so that the largest magnitude of the
32-element block lies in [2^7, 2^8), v = (hi + lo / 16) * 2^s with hi = e4m3(v /
2^s) and lo = e4m3((v / 2^s - hi) * 16).  The claim is that this is exact for
every bf16 value within 2^13 of its block's largest, and that smaller values
keep an error below 2^-20 of that largest.  Here e4m3 (OCP, round to nearest
even, 3 mantissa bits, exponent bias 7, subnormals 2^-9 apart) is written out
from the format's definition and the claim is checked for every finite bf16
value against block maxima from its own binade up to 2^13 above it.
"""
import numpy as np


def e4m3_rne(x):
    """Round float64 values to the nearest e4m3 value (ties to even); |x| < 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # exponent of the binade; below 2^-6 the spacing is that of the subnormals
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)                 # 3 mantissa bits
    q = a / step
    r = np.floor(q)
    frac = q - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0)), r + 1.0, r)
    return np.sign(x) * r * step


def _all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f) & (f != 0)]
    v = f.astype(np.float64)
    return v


def test_e4m3_rounding_against_a_table():
    # every e4m3 value, positive half, from its bit fields
    codes = np.arange(0x7f)                  # 0x7f is NaN
    e = codes >> 3
    m = codes & 7
    table = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))
    assert table.max() == 448.0
    # values round to themselves, midpoints to the even neighbour
    assert np.array_equal(e4m3_rne(table), table)
    mids = (table[1:] + table[:-1]) / 2
    got = e4m3_rne(mids)
    even = np.where(codes[1:] % 2 == 0, table[1:], table[:-1])
    assert np.array_equal(got, even)


def test_two_planes_exact_within_2_13():
    v = _all_bf16()
    ev = np.floor(np.log2(np.abs(v)))
    for d in range(0, 14):                   # block maximum 2^d .. 2^(d+1) above v's binade
        emax = ev + d
        s = emax - 7.0
        xs = v / np.exp2(s)                  # exact: a power of two
        assert np.all(np.abs(xs) < 256.0)
        hi = e4m3_rne(xs)
        rem = (xs - hi) * 16.0
        assert np.all(np.abs(rem) < 448.0)
        lo = e4m3_rne(rem)
        assert np.array_equal(hi + lo / 16.0, xs), f"not exact {d} binades below the block maximum"


def test_two_planes_bound_below_2_13():
    v = _all_bf16()
    ev = np.floor(np.log2(np.abs(v)))
    for d in (14, 16, 20, 30):
        emax = ev + d
        s = emax - 7.0
        xs = v / np.exp2(s)
        hi = e4m3_rne(xs)
        lo = e4m3_rne((xs - hi) * 16.0)
        err = np.abs(hi + lo / 16.0 - xs) * np.exp2(s)
        assert np.all(err < np.exp2(emax - 20.0)), d
