"""Pins of the position-weighted checksum (FreeToken MoE benchmark guide §3.3 properties)."""
import numpy as np

from oracle.checksum import MASK, checksum


def test_small_brute_force():
    data = np.array([3, 0, 7, 255, 1], dtype=np.uint8)
    # N < 2**20 so every byte is sampled: sum (o+1)*b
    assert checksum([data]) == 1 * 3 + 2 * 0 + 3 * 7 + 4 * 255 + 5 * 1


def test_constant_fill_closed_form():
    c, N = 0xA5, 3 * (1 << 20) + 17
    data = np.full(N, c, dtype=np.uint8)
    stride = N // (1 << 20)
    m = (N - 1) // stride + 1          # sampled offsets 0, stride, ..., (m-1)*stride
    want = c * (m + stride * m * (m - 1) // 2) & MASK   # sum of (o+1) over sampled o
    assert checksum([data]) == want


def test_split_independence():
    rng = np.random.default_rng(5)
    flat = rng.integers(0, 256, size=5 * (1 << 20) + 333, dtype=np.uint8)
    h = checksum([flat])
    cuts = [0, 1, 777, 2 * (1 << 20) + 5, 4 * (1 << 20), flat.size]
    pieces = [flat[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    assert checksum(pieces) == h
    assert checksum([flat.reshape(-1)[: flat.size]]) == h


def test_permutation_sensitive():
    rng = np.random.default_rng(9)
    rows = rng.integers(0, 256, size=(8, 4096), dtype=np.uint8)
    h = checksum([rows])
    swapped = rows.copy()
    swapped[[2, 5]] = swapped[[5, 2]]
    assert checksum([swapped]) != h
    # a plain sum would not see the swap
    assert int(rows.sum()) == int(swapped.sum())
