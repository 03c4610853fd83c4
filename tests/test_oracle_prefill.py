"""Pins of the prefill oracle: the buffer is a byte copy of the layer, and the layer FFN
is the routed expert FFN with slot = expert (FreeToken architecture walk-through §5)."""
import numpy as np
import torch

import synth
from oracle import prefill, route
from tests import mxfp4_torch_ref as ref


def test_prefill_layer_is_routed_ffn_on_buffer():
    fmt, H, I, E, k, n = "mxfp4_t", 64, 32, 6, 2, 5
    rows = [synth.expert_rows(fmt, H, I, 0, "pf", e) for e in range(E)]
    nb = len(rows[0])
    host = [[np.concatenate([rows[e][b].numpy() for e in range(E)]).reshape(E, -1)] for b in range(nb)]
    buf = prefill.buffer_after_prefetch(host, 0)
    for b in range(nb):
        assert np.array_equal(buf[b], host[b][0])
        assert buf[b] is not host[b][0]
    logits = synth.router_logits(n, E, 0, "pf").numpy()
    xb = synth.activations(n, H, 0, "pf").numpy().view(np.uint16)
    ids, w, y = prefill.prefill_layer(fmt, H, I, xb, logits, k, buf)
    ids2, w2 = route.topk_softmax(logits, k)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    # the same FFN, one token at a time, from an MXFP4 decoder written apart from the
    # oracle (literal e2m1 table, torch e8m0, torch SiLU), in torch float64
    x64 = torch.from_numpy(xb.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    for t in range(n):
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(k):
            e = int(ids[t, j])
            acc += float(w[t, j]) * ref.output(x64[t:t + 1], [buf[b][e] for b in range(nb)], H, I)[0]
        assert np.allclose(y[t], acc.numpy(), rtol=1e-12, atol=1e-14)
    assert np.abs(y).max() > 0
