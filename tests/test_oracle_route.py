"""Pins of the oracle router: closed forms, tie rule, hand example, library argsort."""
import numpy as np
import torch

from oracle import route


def test_hand_example():
    z = np.array([[1.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    ids, w = route.topk_softmax(z, 2)
    assert ids.tolist() == [[1, 3]]          # equal logits: lower index first
    assert np.allclose(w, [[0.5, 0.5]])
    ids, w = route.topk_softmax(z, 3)
    assert ids.tolist() == [[1, 3, 2]]
    e = np.exp(-1.0)
    assert np.allclose(w[0], [1 / (2 + e), 1 / (2 + e), e / (2 + e)], rtol=1e-14)


def test_topk_equals_stable_argsort_and_weights_sum_to_one():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((50, 32)).astype(np.float32)
    z[3, 7] = z[3, 9]                         # plant a tie
    ids, w = route.topk_softmax(z, 5)
    ref = np.argsort(-z, axis=1, kind="stable")[:, :5]
    assert np.array_equal(ids, ref)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)
    # renormalised softmax over top-k == softmax restricted to the top-k logits
    zk = np.take_along_axis(z.astype(np.float64), ids.astype(np.int64), axis=1)
    sm = np.exp(zk - zk.max(axis=1, keepdims=True))
    assert np.allclose(w, sm / sm.sum(axis=1, keepdims=True), rtol=1e-12)
    # descending weights
    assert (np.diff(w, axis=1) <= 1e-15).all()


def test_router_logits_match_library_matmul():
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal((3, 64)).astype(np.float32)).to(torch.bfloat16)
    wg = torch.from_numpy((0.02 * rng.standard_normal((64, 16))).astype(np.float32)).to(torch.bfloat16)
    z = route.router_logits(x.view(torch.int16).numpy().view(np.uint16), wg.view(torch.int16).numpy().view(np.uint16))
    ref = (x.double() @ wg.double()).float().numpy()
    assert np.array_equal(z, ref)
