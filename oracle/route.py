"""Top-k routing: router logits, softmax over all experts, top-k, renormalise.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the top-k of each MoE layer (FreeToken MoE benchmark guide §4.3
uses bs * topk routed experts) but not the router.  The router taken here is
the plain one: logits = x . Wg, softmax over the E experts, the k largest
probabilities in descending order (equal values: lower expert index first),
weights renormalised to sum to one.

Precision: the logits are computed in float64 from the exact bf16 inputs and
rounded once to float32; the top-k choice is made on those float32 logits, the
precision the GPU side makes it in.  Near-ties (gap of a few float32 ulps) may
legitimately resolve differently on the GPU, whose float32 sum runs in another
order: parity unpinned there.
"""
import numpy as np

from . import decode


def topk_softmax(logits32, k: int):
    """Top-k of float32 logits rows and their renormalised softmax weights (float64)."""
    z = np.asarray(logits32, dtype=np.float32)
    n, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((n, k), dtype=np.int32)
    w = np.empty((n, k), dtype=np.float64)
    for t in range(n):
        order = sorted(range(E), key=lambda e: (-float(z[t, e]), e))[:k]
        ids[t] = order
        zk = z[t, order].astype(np.float64)
        p_all = np.exp(z[t].astype(np.float64) - float(z[t].max()))
        p_all /= p_all.sum()
        pk = p_all[order]
        w[t] = pk / pk.sum()
    return ids, w


def router_logits(x_bits, wg_bits):
    """logits[n, E] = x[n, H] . Wg[H, E] from bf16 bit patterns; float64 sum, rounded once to float32."""
    x = decode.bf16(x_bits)
    wg = decode.bf16(wg_bits)
    return (x @ wg).astype(np.float32)


def route(x_bits, wg_bits, k: int):
    """Route tokens: returns (ids int32 [n, k], w float64 [n, k], logits float32 [n, E])."""
    z = router_logits(x_bits, wg_bits)
    ids, w = topk_softmax(z, k)
    return ids, w, z
