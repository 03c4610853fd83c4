"""GPU parity of prefill: whole-layer streaming into a two-deep buffer and the MXFP4
grouped expert FFN (MFMA), against the oracle."""
import numpy as np
import pytest
import torch

import offloaded_expert_slot_amd as oes
import synth
from oracle import ffn as offn
from oracle import route as oroute
from synth.workloads import WORKLOADS, Workload, make_host_banks
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _layers(w, hb, depth=2, layers=1):
    sc = oes.schema_make(w.fmt, layers, w.E, w.H, w.I)
    L = oes.Layers(sc, depth, 0)
    for layer in range(layers):
        for b, t in enumerate(hb.banks):
            L.set_source(b, layer, t)   # one host bank reused under every layer id
    return L


def _run_ffn(L, layer, x, ids, w):
    n, k = ids.shape
    y = torch.empty((n, x.shape[1]), dtype=torch.int16, device=G.dev())
    ws = torch.empty(L.ffn_workspace_bytes(n, k), dtype=torch.uint8, device=G.dev())
    L.ffn(layer, x, ids, w, y, ws)
    return y


def _oracle_rows(hb, sel_ids):
    cache = {}

    def rows(e):
        if e not in cache:
            cache[e] = [hb.row(b, e).numpy() for b in range(len(hb.banks))]
        return cache[e]
    return rows


@pytest.mark.parametrize("H,I,E,k,n,hot", [
    (128, 192, 16, 4, 100, None),       # ragged groups, several feature tiles
    (192, 128, 12, 2, 70, None),        # E not a multiple of 8: plain block mapping
    (128, 128, 8, 2, 300, 3),           # one expert gets every token: 3 passes of 128 rows
    (64, 128, 1024, 4, 300, None),      # dispatch order ranked over 1024 experts, one quad of K
    (64, 64, 1100, 2, 200, None),       # past 1024 experts: dispatch in index order
])
def test_prefill_ffn_small(H, I, E, k, n, hot):
    _case(f"prefill ffn H={H} I={I} E={E} k={k} n={n} hot={hot}")
    w = Workload(f"pf-{H}-{I}-{E}", "mxfp4_t", L=1, E=E, k=k, H=H, I=I, S=0)
    hb = make_host_banks(w)
    L = _layers(w, hb)
    L.prefetch(0)
    logits = synth.router_logits(n, E, 0, w.name).numpy()
    ids, wts = oroute.topk_softmax(logits, k)
    if hot is not None:
        ids[:, 0] = hot
        ids[:, 1] = np.where(ids[:, 1] == hot, (hot + 1) % E, ids[:, 1])
    ids[5, -1] = -1 if hot is None else ids[5, -1]   # an invalid pair is skipped
    x = synth.activations(n, H, 0, w.name).to(G.dev())
    y = _run_ffn(L, 0, x, torch.from_numpy(ids.astype(np.int32)).to(G.dev()),
                 torch.from_numpy(wts.astype(np.float32)).to(G.dev()))
    torch.cuda.synchronize()
    rows = _oracle_rows(hb, None)
    ref = offn.expert_ffn("mxfp4_t", H, I, G.bits16(x), ids, wts.astype(np.float32).astype(np.float64), rows)
    err = offn.rel_l2(G.bf16_tensor_to_f64(y), ref)
    print(f"  rel_l2={err:.3e}")
    assert err <= 3e-2
    # the two e4m3 planes hold each bf16 activation exactly and the fp4 weights
    # enter the MFMA as they are, so what is left is the bf16 rounding of h, of
    # each pair's o and of y (about 2^-9 relative each; 2.4e-3 measured): a plane
    # lost or mis-scaled costs above 1e-2
    assert err <= 4e-3
    # the buffer holds the layer's bytes
    for b in range(len(hb.banks)):
        assert torch.equal(L.buffer_view(0, b).cpu(), hb.banks[b])


def test_prefill_ffn_edges():
    """n = 0 launches nothing; one token with one pair (a single row padded to a full
    m-tile); skipped pairs (-1 and ids >= E) and a token with every pair skipped (y = 0)."""
    H, I, E = 128, 192, 16
    w = Workload(f"pf-edge-{H}-{I}-{E}", "mxfp4_t", L=1, E=E, k=2, H=H, I=I, S=0)
    hb = make_host_banks(w)
    L = _layers(w, hb)
    L.prefetch(0)
    dev = G.dev()
    _case("prefill ffn n=0")
    y0 = torch.full((0, H), 7, dtype=torch.int16, device=dev)
    L.ffn(0, torch.empty((0, H), dtype=torch.int16, device=dev), torch.empty((0, 2), dtype=torch.int32, device=dev),
          torch.empty((0, 2), dtype=torch.float32, device=dev), y0,
          torch.empty(max(16, L.ffn_workspace_bytes(0, 2)), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    rows = _oracle_rows(hb, None)
    for n, k in ((1, 1), (40, 2)):
        _case(f"prefill ffn edges n={n} k={k}")
        logits = synth.router_logits(n, E, 1, w.name).numpy()
        ids, wts = oroute.topk_softmax(logits, k)
        ids = ids.astype(np.int32)
        if n > 1:
            ids[3, :] = -1           # every pair skipped
            ids[4, 0] = E            # out of range: skipped
            ids[5, 1] = 1 << 30
        x = synth.activations(n, H, 1, w.name).to(dev)
        y = _run_ffn(L, 0, x, torch.from_numpy(ids).to(dev), torch.from_numpy(wts.astype(np.float32)).to(dev))
        torch.cuda.synchronize()
        oids = np.where((ids >= 0) & (ids < E), ids, -1)
        ref = offn.expert_ffn("mxfp4_t", H, I, G.bits16(x), oids, wts.astype(np.float32).astype(np.float64), rows)
        got = G.bf16_tensor_to_f64(y)
        if n > 1:
            assert not got[3].any() and not ref[3].any()
        err = offn.rel_l2(got, ref)
        print(f"  rel_l2={err:.3e}")
        assert err <= 4e-3


def test_prefill_ffn_activation_ranges():
    """The two e4m3 activation planes across value ranges: a zero row, a constant row,
    rows whose 32-element blocks span 2^30 (beyond the 2^13 exact range), tiny and
    large magnitudes; the error stays at the bf16 rounding of h, o and y."""
    H, I, E, k, n = 192, 128, 8, 2, 48
    _case(f"prefill ffn activation ranges H={H} I={I} E={E} k={k} n={n}")
    w = Workload(f"pf-rng-{H}-{I}-{E}", "mxfp4_t", L=1, E=E, k=k, H=H, I=I, S=0)
    hb = make_host_banks(w)
    L = _layers(w, hb)
    L.prefetch(0)
    logits = synth.router_logits(n, E, 0, w.name).numpy()
    ids, wts = oroute.topk_softmax(logits, k)
    rng = np.random.default_rng(7)
    xf = rng.standard_normal((n, H))
    xf[0] = 0.0
    xf[1] = 1.0
    for r in (2, 3, 4):   # wide dynamic range inside every block
        xf[r] = np.sign(rng.standard_normal(H)) * np.exp2(rng.uniform(-20.0, 10.0, H))
    xf[5] = rng.standard_normal(H) * 1e-30
    xf[6] = rng.standard_normal(H) * 3e2
    xf[7, ::32] = 5e2      # one large element per block, the rest N(0, 1)
    x = torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16).view(torch.int16).to(G.dev())
    y = _run_ffn(L, 0, x, torch.from_numpy(ids.astype(np.int32)).to(G.dev()),
                 torch.from_numpy(wts.astype(np.float32)).to(G.dev()))
    torch.cuda.synchronize()
    rows = _oracle_rows(hb, None)
    ref = offn.expert_ffn("mxfp4_t", H, I, G.bits16(x), ids, wts.astype(np.float32).astype(np.float64), rows)
    got = G.bf16_tensor_to_f64(y)
    assert np.isfinite(got).all()
    for r in range(n):
        e = offn.rel_l2(got[r:r + 1], ref[r:r + 1])
        assert e <= 6e-3, f"row {r}: rel_l2 {e:.3e}"
    err = offn.rel_l2(got, ref)
    print(f"  rel_l2={err:.3e}")
    assert err <= 4e-3


def _rotated_banks(hb, shift):
    """Pinned copies of layer 0's banks with the expert rows rotated: row e holds
    layer 0's expert (e + shift) % E in every bank (distinct bytes per layer, valid
    weights, and an oracle that is layer 0's with the ids shifted)."""
    out = []
    for t, rb in zip(hb.banks, hb.row_bytes):
        r = torch.empty(t.numel(), dtype=torch.uint8, pin_memory=True)
        r.view(hb.E, rb).copy_(torch.roll(t.view(hb.E, rb), -shift, dims=0))
        out.append(r)
    return out


@pytest.mark.timeout(900)
def test_prefill_full_size_streamed():
    """The prefill workload at full size (H = I = 2880, 128 experts, top-4, 2048
    tokens): four layers with distinct bytes stream through the two-deep buffer
    on a copy stream while the grouped FFN runs on the compute stream, and every
    output row of every layer is checked against the oracle.

    Odd layers run their FFN 60 times (longer than the next layer's 1.69 GB copy),
    so a prefetch that did not wait for the buffer's release would overwrite the
    weights under the later launches; layer 1 is enqueued long before its copy
    lands, so an FFN that did not wait for its copy would read the previous
    bytes.  The first and the last launch of each layer are both checked."""
    w = WORKLOADS["mxfp4_prefill"]
    layers, repeats = 4, (1, 60, 1, 60)
    _case(f"prefill full size streamed H={w.H} I={w.I} E={w.E} k={w.k} n={w.tokens} layers={layers}")
    dev = G.dev()
    hb = make_host_banks(w)
    banks = [hb.banks] + [_rotated_banks(hb, l) for l in range(1, layers)]
    for l in range(1, layers):
        assert not torch.equal(banks[l][0], banks[0][0])
    sc = oes.schema_make(w.fmt, layers, w.E, w.H, w.I)
    Lo = oes.Layers(sc, 2, 0)
    for l in range(layers):
        for b, t in enumerate(banks[l]):
            Lo.set_source(b, l, t)
    logits = synth.router_logits(w.tokens, w.E, 0, w.name)
    ids = torch.empty((w.tokens, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.tokens, w.k), dtype=torch.float32, device=dev)
    oes.route_logits(logits.to(dev), w.k, ids, wts)
    x = synth.activations(w.tokens, w.H, 0, w.name).to(dev)
    ws = torch.empty(Lo.ffn_workspace_bytes(w.tokens, w.k), dtype=torch.uint8, device=dev)
    first = [torch.empty((w.tokens, w.H), dtype=torch.int16, device=dev) for _ in range(layers)]
    last = [torch.empty((w.tokens, w.H), dtype=torch.int16, device=dev) for _ in range(layers)]
    spare = torch.empty((w.tokens, w.H), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    oids, ow = oroute.topk_softmax(logits.numpy(), w.k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert len(set(oids.ravel().tolist())) == w.E          # every expert is active
    copy_stream, comp = torch.cuda.Stream(), torch.cuda.current_stream()
    Lo.prefetch(0, copy_stream)
    for l in range(layers):
        if l + 1 < layers:
            Lo.prefetch(l + 1, copy_stream)
        for r in range(repeats[l]):
            out = first[l] if r == 0 else (last[l] if r == repeats[l] - 1 else spare)
            Lo.ffn(l, x, ids, wts, out, ws, comp)
    torch.cuda.synchronize()
    # the buffers hold the last two layers' bytes
    for l in (layers - 2, layers - 1):
        for b in range(len(hb.banks)):
            assert torch.equal(Lo.buffer_view(l % 2, b).cpu(), banks[l][b]), (l, b)
    # layer l's expert e is layer 0's expert (e + l) % E, so one oracle call over the
    # four layers' tokens stacked (ids shifted per layer) gives every layer's y
    ids_all = np.concatenate([(oids + l) % w.E for l in range(layers)])
    w_all = np.tile(ow.astype(np.float32).astype(np.float64), (layers, 1))
    x_bits = G.bits16(x)
    rows = _oracle_rows(hb, None)
    ref = offn.expert_ffn("mxfp4_t", w.H, w.I, np.tile(x_bits, (layers, 1)), ids_all, w_all, rows)
    n = w.tokens
    for l in range(layers):
        ref_l = ref[l * n:(l + 1) * n]
        for tag, y in (("first", first[l]), ("last", last[l])):
            if tag == "last" and repeats[l] == 1:
                continue
            got = G.bf16_tensor_to_f64(y)
            err = offn.rel_l2(got, ref_l)
            worst = max(offn.rel_l2(got[i:i + 1], ref_l[i:i + 1]) for i in range(n))
            print(f"  layer {l} {tag}: rel_l2={err:.3e} worst token {worst:.3e}", flush=True)
            assert err <= 3e-2 and worst <= 3e-2
            # bf16 rounding of h, o and y only (the activation planes are exact)
            assert err <= 5e-3 and worst <= 1e-2
        if repeats[l] > 1:   # every launch of a layer gives the same bits
            assert torch.equal(first[l], last[l])
    Lo.close()


def test_layer_streaming_double_buffer():
    """Four layers through two buffers: prefetch l+1 on a side stream while layer l computes."""
    H, I, E, k, n, layers = 128, 128, 16, 2, 64, 4
    _case("layer streaming 4 layers depth 2")
    w = Workload("pf-stream", "mxfp4_t", L=1, E=E, k=k, H=H, I=I, S=0)
    hbs = [make_host_banks(w, seed=s) for s in range(layers)]   # distinct bytes per layer
    sc = oes.schema_make(w.fmt, layers, E, H, I)
    Lo = oes.Layers(sc, 2, 0)
    for layer in range(layers):
        for b, t in enumerate(hbs[layer].banks):
            Lo.set_source(b, layer, t)
    copy_stream = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    logits = synth.router_logits(n, E, 0, w.name).numpy()
    ids, wts = oroute.topk_softmax(logits, k)
    d_ids = torch.from_numpy(ids.astype(np.int32)).to(G.dev())
    d_w = torch.from_numpy(wts.astype(np.float32)).to(G.dev())
    x = synth.activations(n, H, 0, w.name).to(G.dev())
    ws = torch.empty(Lo.ffn_workspace_bytes(n, k), dtype=torch.uint8, device=G.dev())
    ys = [torch.empty((n, H), dtype=torch.int16, device=G.dev()) for _ in range(layers)]
    torch.cuda.synchronize()
    Lo.prefetch(0, copy_stream)
    for layer in range(layers):
        if layer + 1 < layers:
            Lo.prefetch(layer + 1, copy_stream)
        Lo.ffn(layer, x, d_ids, d_w, ys[layer], ws, comp)
    torch.cuda.synchronize()
    for layer in range(layers):
        hb = hbs[layer]
        ref = offn.expert_ffn("mxfp4_t", H, I, G.bits16(x), ids, wts.astype(np.float32).astype(np.float64),
                              lambda e: [hb.row(b, e).numpy() for b in range(len(hb.banks))])
        err = offn.rel_l2(G.bf16_tensor_to_f64(ys[layer]), ref)
        print(f"  layer {layer} rel_l2={err:.3e}")
        assert err <= 4e-3
    # an ffn on a layer that is not resident is refused
    with pytest.raises(oes.OesError):
        Lo.ffn(0, x, d_ids, d_w, ys[0], ws, comp)
