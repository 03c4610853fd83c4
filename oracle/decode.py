"""Bit-field decoders for the element formats the banks hold.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These are written from the public format definitions (IEEE binary16, the
bfloat16 truncation of binary32, OCP 8-bit e4m3 "fn", the OCP microscaling
e8m0 scale and e2m1 element), not from any table shared with the GPU code.
Every decoder returns float64.
"""
import numpy as np


def bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64: the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16(bits):
    """IEEE binary16 bit patterns -> float64, from sign / 5-bit exponent / 10-bit mantissa."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    sub = s * (m / 1024.0) * 2.0 ** -14
    norm = s * (1.0 + m / 1024.0) * np.power(2.0, (e - 15).astype(np.float64))
    out = np.where(e == 0, sub, norm)
    out = np.where((e == 31) & (m == 0), s * np.inf, out)
    out = np.where((e == 31) & (m != 0), np.nan, out)
    return out


def e4m3(bits):
    """OCP e4m3 'fn' bytes -> float64.

    Sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0
    is subnormal (m/8 * 2**-6); there is no infinity and S.1111.111 is NaN;
    the largest finite value is 448.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    sub = s * (m / 8.0) * 2.0 ** -6
    norm = s * (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    out = np.where(e == 0, sub, norm)
    return np.where((e == 15) & (b & 7 == 7), np.nan, out)


def e8m0(bits):
    """OCP e8m0 scale bytes -> float64: 2**(b - 127); 0xFF is NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.float64)
    return np.where(b == 255, np.nan, np.power(2.0, b - 127.0))


def e2m1(codes):
    """OCP e2m1 4-bit codes (values 0..15) -> float64.

    Sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0; exponent 0 is
    subnormal (0 or 0.5).  Magnitudes are {0, .5, 1, 1.5, 2, 3, 4, 6}.
    """
    c = np.asarray(codes).astype(np.int64)
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.power(2.0, (e - 1).astype(np.float64)))
    return s * mag


def fp4x2_unpack(packed):
    """Bytes holding two e2m1 codes -> codes along the last axis, twice as long.

    Element 2j sits in the low nibble and element 2j+1 in the high nibble of
    byte j (a reading: the pages say only "packed codes").  Parity unpinned
    beyond the round-trip pin against the fp32 weights the codes were made from.
    """
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def q4x2_unpack(packed):
    """GGUF Q4_0 code bytes -> 4-bit codes in element order, along the last axis.

    GGUF block_q4_0: 32 elements per block; of the block's 16 code bytes, byte j
    holds element j in its low nibble and element j + 16 in its high nibble.
    """
    p = np.asarray(packed, dtype=np.uint8)
    blocks = p.reshape(p.shape[:-1] + (p.shape[-1] // 16, 16))
    codes = np.concatenate([blocks & 0xF, blocks >> 4], axis=-1)       # [..., blocks, 32]
    return codes.reshape(p.shape[:-1] + (2 * p.shape[-1],))


def q4_0(codes):
    """GGUF Q4_0 4-bit codes -> the integers q - 8 (the weight before its block scale d)."""
    return np.asarray(codes).astype(np.int64).astype(np.float64) - 8.0


def via_table(fn, codes, ncodes):
    """fn applied to integer codes by evaluating fn once on every possible code.

    Same values as fn(codes); used for large arrays of 4- and 8-bit codes.
    """
    table = fn(np.arange(ncodes))
    return table[np.asarray(codes).astype(np.intp)]
