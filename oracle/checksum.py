"""Position-weighted sampled checksum of a bank.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FreeToken MoE benchmark guide §3.3: the checksum samples about a million bytes
of each bank, weighting each sampled byte by its global byte offset so that a
reordering of experts changes the result; offsets run across the per-layer
tensors as if they were concatenated, so the value does not depend on how the
bank is split, and no concatenated copy is made.

The exact fold is not on the page; the reading taken (parity unpinned against
the page) is

    stride = max(1, N // 2**20)
    h      = sum over o = 0, stride, 2*stride, ... < N of (o + 1) * byte[o]   mod 2**64
"""
import numpy as np

MASK = (1 << 64) - 1


def checksum(pieces):
    """Checksum of a bank given as a list of byte arrays, in order, as one flat sequence."""
    arrs = [np.asarray(p).reshape(-1).view(np.uint8) for p in pieces]
    total = sum(a.size for a in arrs)
    stride = max(1, total // (1 << 20))
    h = 0
    base = 0
    for a in arrs:
        # first sampled global offset inside this piece
        first = (-base) % stride
        offs = np.arange(first, a.size, stride, dtype=np.int64)
        if offs.size:
            weights = (offs + base + 1).astype(object)
            vals = a[offs].astype(object)
            h = (h + int(np.sum(weights * vals))) & MASK
        base += a.size
    return h
