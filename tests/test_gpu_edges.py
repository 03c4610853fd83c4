"""Edge cases of the step on the GPU, against the oracle: empty steps, the
largest slot pool and expert count the remap supports, the largest top-k and
hidden size of the decode FFN, and an FFN whose pairs are all skipped."""
import numpy as np
import pytest
import torch

import offloaded_expert_slot_amd as oes
import synth
from oracle import copy as ocopy
from oracle import ffn as offn
from oracle import route as oroute
from oracle.lru import OK, SlotTable
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def test_empty_steps():
    """n = 0 through every step call: nothing computed; the remap still advances
    the clock (a step with no requests), as the oracle does."""
    _case("empty steps")
    fmt, L, E, H, I, S, k = "bf16", 1, 8, 64, 64, 4, 2
    banks = {0: G.make_banks(fmt, E, H, I, tag="edge-empty")}
    c = G.make_cache(fmt, L, E, H, I, S, banks)
    t = SlotTable(S, L, E)
    dev = G.dev()
    ids = torch.empty((0, k), dtype=torch.int32, device=dev)
    w = torch.empty((0, k), dtype=torch.float32, device=dev)
    x = torch.empty((0, H), dtype=torch.int16, device=dev)
    wg = synth.router_weight(H, E, 0, "edge-empty").to(dev)
    ws = torch.empty(max(16, oes.route_workspace_bytes(0, H, E)), dtype=torch.uint8, device=dev)
    oes.route(x, wg, k, ids, w, ws)
    slots = torch.empty_like(ids)
    for _ in range(2):
        c.ensure_experts(0, ids, slots)
        c.copy_missing()
        c.expert_ffn(x, slots, w, torch.empty((0, H), dtype=torch.int16, device=dev),
                     torch.empty(16, dtype=torch.uint8, device=dev))
        assert t.ensure(0, np.zeros((0, k), dtype=np.int32)).status == OK
    torch.cuda.synchronize()
    c.check()
    owner, stamp, clock = c.get_state()
    assert owner.tolist() == t.owner.tolist() and stamp.tolist() == t.stamp.tolist() and clock == t.clock == 2
    assert c.get_misses() == []
    cpu = oes.CpuMoe(oes.schema_make(fmt, L, E, H, I), 2)
    cpu.run(0, np.zeros((0, H), np.uint16), np.zeros((0, k), np.int32), np.zeros((0, k), np.int32),
            np.zeros((0, k), np.float32), np.zeros((0, H), np.float32))
    cpu.close()


def test_largest_pool_and_expert_count():
    """OES_MAX_SLOTS slots over three layers of 2048 experts: filling the pool,
    hits, and steps of 2048 misses that evict a whole layer; slot maps, table and
    slot bytes against the oracle."""
    _case("pool 4096 slots, E=2048, L=3")
    fmt, L, E, H, I = "bf16", 3, 2048, 64, 32
    S = oes.MAX_SLOTS
    banks = {layer: G.make_banks(fmt, E, H, I, layer=layer, tag="edge-max") for layer in range(L)}
    c = G.make_cache(fmt, L, E, H, I, S, banks)
    c.fill_slots(0xA5)
    host = G.oracle_host(banks, L, 2)
    mirror = [np.full((S, rb), 0xA5, dtype=np.uint8) for rb in banks[0].row_bytes]
    t = SlotTable(S, L, E)
    rng = np.random.default_rng(41)
    plan = [(0, np.arange(E)), (1, np.arange(E)), (0, rng.choice(E, 64, replace=False)),
            (2, rng.permutation(E)), (1, rng.choice(E, 96, replace=False)), (0, rng.choice(E, 5, replace=False)),
            (2, rng.choice(E, 32, replace=False))]
    for step, (layer, e) in enumerate(plan):
        k = 32 if len(e) % 32 == 0 else 1
        ids = e.astype(np.int32).reshape(-1, k)
        d_ids = torch.from_numpy(ids).to(G.dev())
        d_slots = torch.empty_like(d_ids)
        c.ensure_experts(layer, d_ids, d_slots)
        c.copy_missing()
        r = t.ensure(layer, ids)
        assert r.status == OK
        ocopy.copy_missing(r.misses, host, mirror, E)
        torch.cuda.synchronize()
        c.check()
        assert np.array_equal(d_slots.cpu().numpy(), r.slot_ids), step
        assert c.get_misses() == r.misses, step
        owner, stamp, clock = c.get_state()
        assert owner.tolist() == t.owner.tolist() and stamp.tolist() == t.stamp.tolist(), step
        for b in range(2):
            assert np.array_equal(G.slot_bytes(c, b), mirror[b]), (step, b)


def test_route_and_ffn_at_top32_and_largest_hidden():
    """k = 32 (the largest top-k) at H = 16384 (the largest hidden size of the
    decode FFN): router picks and FFN against the oracle."""
    fmt, E, H, I, k, n = "bf16", 40, 16384, 128, 32, 2
    _case(f"route + ffn H={H} k={k}")
    dev = G.dev()
    x = synth.activations(n, H, 0, "edge-k32").to(dev)
    wg = synth.router_weight(H, E, 0, "edge-k32").to(dev)
    ids = torch.empty((n, k), dtype=torch.int32, device=dev)
    w = torch.empty((n, k), dtype=torch.float32, device=dev)
    oes.route(x, wg, k, ids, w, torch.empty(oes.route_workspace_bytes(n, H, E), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    oids, ow, _ = oroute.route(G.bits16(x), G.bits16(wg), k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=2e-4, atol=1e-6)
    banks = {0: G.make_banks(fmt, E, H, I, tag="edge-k32")}
    c = G.make_cache(fmt, 1, E, H, I, E, banks)
    c.load_rows(list(range(E)), list(range(E)))   # slot s holds expert s
    y = torch.empty((n, H), dtype=torch.int16, device=dev)
    c.expert_ffn(x, ids, w, y, torch.empty(c.ffn_workspace_bytes(n, k), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    c.check()
    hb = banks[0]
    ref = offn.expert_ffn(fmt, H, I, G.bits16(x), oids, ow.astype(np.float32).astype(np.float64),
                          lambda s: [hb.row(b, s).numpy() for b in range(len(hb.banks))])
    err = offn.rel_l2(G.bf16_tensor_to_f64(y), ref)
    print(f"  rel_l2={err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "q4_0"])
def test_ffn_with_every_pair_skipped(fmt):
    """slot -1 everywhere (a hybrid step that fetched nothing): y is exactly zero."""
    _case(f"ffn all skipped {fmt}")
    E, H, I, k, n = 4, 256, 256, 3, 3
    banks = {0: G.make_banks(fmt, E, H, I, tag="edge-skip")}
    c = G.make_cache(fmt, 1, E, H, I, E, banks)
    dev = G.dev()
    x = synth.activations(n, H, 0, "edge-skip").to(dev)
    slots = torch.full((n, k), -1, dtype=torch.int32, device=dev)
    w = torch.full((n, k), 1.0 / k, dtype=torch.float32, device=dev)
    y = torch.full((n, H), 0x3f80, dtype=torch.int16, device=dev)
    c.expert_ffn(x, slots, w, y, torch.empty(c.ffn_workspace_bytes(n, k), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    c.check()
    assert (y == 0).all()
