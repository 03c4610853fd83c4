"""GPU parity against the oracle at the decode workloads' full sizes.

For each decode workload (tiny bf16 H=256, bf16 H=2048, fp8-block H=4096, nvfp4
H=7168, GGUF Q4_0 H=2048; full expert count, full slot pool with every slot
owned by another layer):

* every copy-sweep row (each bs x miss rate of the workload, fused and per-bank)
  runs through ensure_experts + copy_missing exactly as the benchmark times it;
  the slot map, miss list and owners must equal the oracle LRU's, every touched
  slot must hold the host row byte for byte in every bank, and sampled
  untouched slots must still hold the sentinel;
* the decode step (route -> ensure -> copy -> FFN) at every miss rate of the
  workload must match the oracle: routed ids, slot map and misses exactly, y to
  the relative-L2 bound of the format;
* the batched FFN on routed ids is checked on every token.
"""
import time

import numpy as np
import pytest
import torch

import offloaded_expert_slot_amd as oes
import synth
from oracle import ffn as offn
from oracle import formulas
from oracle import route as oroute
from oracle.lru import OK, SlotTable
from synth.workloads import WORKLOADS, make_host_banks
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

_STATE = {}          # workload name -> its host banks, cache and device copy of the banks


@pytest.fixture(scope="module", autouse=True)
def _free_workloads():
    yield
    for st in _STATE.values():
        st["c"].close()
    _STATE.clear()
    torch.cuda.empty_cache()


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _setup(name):
    """Host banks (layer 0) and a cache of the workload, built once per module run."""
    if name not in _STATE:
        w = WORKLOADS[name]
        hb = make_host_banks(w)
        sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
        c = oes.Cache(sc, w.S, 0)
        for b, t in enumerate(hb.banks):
            c.set_source(b, 0, t)
        _STATE[name] = dict(w=w, hb=hb, c=c, sc=sc)
    st = _STATE[name]
    st["c"].set_option(oes.OPT_FUSED_COPY, 1)
    st["c"].set_option(oes.OPT_FFN_PATH, oes.FFN_AUTO)
    return st["w"], st["hb"], st["c"]


def _host_on_device(name):
    """The layer-0 host banks copied to the device once ([E, row_bytes] each), for byte compares."""
    st = _STATE[name]
    if "hb_dev" not in st:
        hb = st["hb"]
        st["hb_dev"] = [t.to(G.dev()).view(hb.E, rb) for t, rb in zip(hb.banks, hb.row_bytes)]
    return st["hb_dev"]


DECODE = ("bf16_tiny", "bf16_h2048", "fp8_h4096", "nvfp4_h7168", "q4_0_h2048")
# every (bs, miss rate) row of every decode workload, fused and per-bank, grouped by workload
SWEEP_ROWS = [(name, bs, mr, fused) for name in DECODE for bs in WORKLOADS[name].batches
              for mr in WORKLOADS[name].miss_rates for fused in (1, 0)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,bs,mr,fused", SWEEP_ROWS)
def test_copy_sweep_row(name, bs, mr, fused):
    w, hb, c = _setup(name)
    _case(f"copy sweep {name} bs={bs} mr={mr} fused={fused}")
    c.set_option(oes.OPT_FUSED_COPY, fused)
    ids = synth.synthetic_ids(bs, w.k, w.E, 0, w.name).numpy()
    active = formulas.active_unique(bs, w.k, w.E)
    assert len(set(ids.ravel().tolist())) == active
    m = formulas.num_misses(active, mr)
    owner, stamp, clock, _ = synth.forced_miss_state(w.S, w.E, 0, ids, m)
    c.fill_slots(0xA5)
    c.set_state(owner, stamp, clock)
    d_ids = torch.from_numpy(ids).to(G.dev())
    d_slots = torch.empty_like(d_ids)
    c.ensure_experts(0, d_ids, d_slots)
    c.copy_missing()
    torch.cuda.synchronize()
    c.check()
    t = SlotTable(w.S, w.L, w.E)
    t.set_state(owner, stamp, clock)
    r = t.ensure(0, ids)
    assert r.status == OK and len(r.misses) == m
    assert np.array_equal(d_slots.cpu().numpy(), r.slot_ids)
    assert c.get_misses() == r.misses
    got_owner, got_stamp, got_clock = c.get_state()
    assert np.array_equal(got_owner, t.owner) and np.array_equal(got_stamp, t.stamp) and got_clock == t.clock
    touched = sorted(s_ for s_, _ in r.misses)
    rng = np.random.default_rng(0)
    untouched = [int(s_) for s_ in rng.choice(w.S, size=min(w.S, 64), replace=False) if int(s_) not in set(touched)]
    hb_dev = _host_on_device(name)
    if touched:
        sl = torch.tensor([s_ for s_, _ in r.misses], dtype=torch.long, device=G.dev())
        ex = torch.tensor([fid % w.E for _, fid in r.misses], dtype=torch.long, device=G.dev())
    for b in range(len(hb.banks)):
        view = c.slot_bank_view(b)
        if touched:   # every byte of every missed row of this bank
            assert torch.equal(view[sl], hb_dev[b][ex]), (b, name, bs, mr)
        if untouched:
            assert bool((view[torch.tensor(untouched, device=G.dev())] == 0xA5).all()), (b, untouched)
    c.set_option(oes.OPT_FUSED_COPY, 1)


# the decode step at every miss rate of each workload: bs=1, and bs 1 and 4 for the tiny one
DECODE_STEPS = [(name, bs, mr) for name in DECODE for bs in ((1, 4) if name == "bf16_tiny" else (1,))
                for mr in WORKLOADS[name].miss_rates]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,bs,mr", DECODE_STEPS)
def test_decode_step(name, bs, mr):
    w, hb, c = _setup(name)
    _case(f"decode step {name} bs={bs} mr={mr}")
    dev = G.dev()
    x = synth.activations(bs, w.H, 0, w.name).to(dev)
    wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
    ids = torch.empty((bs, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((bs, w.k), dtype=torch.float32, device=dev)
    oes.route(x, wg, w.k, ids, wts, torch.empty(oes.route_workspace_bytes(bs, w.H, w.E), dtype=torch.uint8,
                                                  device=dev))
    torch.cuda.synchronize()
    # the routed ids are the oracle router's; the GPU router must agree on them
    routed, ow, _ = oroute.route(G.bits16(x), G.bits16(wg), w.k)
    assert np.array_equal(ids.cpu().numpy(), routed)
    np.testing.assert_allclose(wts.cpu().numpy(), ow, rtol=2e-4, atol=1e-6)
    m = formulas.num_misses(len(set(routed.ravel().tolist())), mr)
    owner, stamp, clock, pre = synth.forced_miss_state(w.S, w.E, 0, routed, m)
    c.set_state(owner, stamp, clock)
    if pre:
        c.load_rows([p[0] for p in pre], [p[1] for p in pre])
    slot_ids = torch.empty_like(ids)
    y = torch.empty((bs, w.H), dtype=torch.int16, device=dev)
    ws = torch.empty(c.ffn_workspace_bytes(bs, w.k), dtype=torch.uint8, device=dev)
    c.ensure_experts(0, ids, slot_ids)
    c.copy_missing()
    c.expert_ffn(x, slot_ids, wts, y, ws)
    torch.cuda.synchronize()
    c.check()
    t = SlotTable(w.S, w.L, w.E)
    t.set_state(owner, stamp, clock)
    r = t.ensure(0, routed)
    assert np.array_equal(slot_ids.cpu().numpy(), r.slot_ids)
    assert c.get_misses() == r.misses and len(r.misses) == m
    # the oracle reads each slot's expert from the host banks by the slot's owner
    ref = offn.expert_ffn(w.fmt, w.H, w.I, G.bits16(x), r.slot_ids, ow,
                          lambda s: [hb.row(b, int(t.owner[s]) % w.E).numpy() for b in range(len(hb.banks))])
    err = offn.rel_l2(G.bf16_tensor_to_f64(y), ref)
    print(f"  rel_l2={err:.3e}")
    assert err <= (3e-2 if w.fmt in ("nvfp4", "q4_0") else 1e-2)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", ["per_pair", "grouped"])
@pytest.mark.parametrize("name,bs", [("bf16_h2048", 8), ("bf16_h2048", 32), ("fp8_h4096", 16),
                                     ("nvfp4_h7168", 4), ("q4_0_h2048", 8)])
def test_decode_ffn_batched(name, bs, path):
    """Batched FFN on routed ids (every slot foreign, so every routed expert is
    copied in first), on both FFN paths; the oracle checks every token."""
    w, hb, c = _setup(name)
    _case(f"ffn {name} bs={bs} path={path}")
    c.set_option(oes.OPT_FFN_PATH, oes.FFN_GROUPED if path == "grouped" else oes.FFN_PER_PAIR)
    dev = G.dev()
    x = synth.activations(bs, w.H, 0, w.name, step=7).to(dev)
    wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
    oids, ow, _ = oroute.route(G.bits16(x), G.bits16(wg), w.k)
    ids = torch.from_numpy(oids).to(dev)
    wts = torch.from_numpy(ow.astype(np.float32)).to(dev)
    owner, stamp, clock = synth.foreign_state(w.S, w.E)
    c.set_state(owner, stamp, clock)
    slot_ids = torch.empty_like(ids)
    y = torch.empty((bs, w.H), dtype=torch.int16, device=dev)
    ws = torch.empty(c.ffn_workspace_bytes(bs, w.k), dtype=torch.uint8, device=dev)
    c.ensure_experts(0, ids, slot_ids)
    c.copy_missing()
    c.expert_ffn(x, slot_ids, wts, y, ws)
    torch.cuda.synchronize()
    c.check()
    t = SlotTable(w.S, w.L, w.E)
    t.set_state(owner, stamp, clock)
    r = t.ensure(0, oids)
    assert np.array_equal(slot_ids.cpu().numpy(), r.slot_ids)
    ref = offn.expert_ffn(w.fmt, w.H, w.I, G.bits16(x), r.slot_ids, ow.astype(np.float32).astype(np.float64),
                          lambda s: [hb.row(b, int(t.owner[s]) % w.E).numpy() for b in range(len(hb.banks))])
    got = G.bf16_tensor_to_f64(y)
    err = offn.rel_l2(got, ref)
    worst = max(offn.rel_l2(got[i:i + 1], ref[i:i + 1]) for i in range(bs))
    print(f"  rel_l2={err:.3e} worst token {worst:.3e}")
    assert worst <= (3e-2 if w.fmt in ("nvfp4", "q4_0") else 1e-2)
    assert err <= (3e-2 if w.fmt in ("nvfp4", "q4_0") else 1e-2)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("max_fetch,frac", [(-1, 0.3), (5, -1.0), (-1, -1.0)])
def test_hybrid_step_bs8(max_fetch, frac):
    """ensure_experts_hybrid at full size (bf16 H=2048, every slot foreign): the
    fetched misses are copied and the FFN runs on the resident pairs only; the
    overflow pairs map to -1 (the CPU executor's share, not computed here)."""
    w, hb, c = _setup("bf16_h2048")
    _case(f"hybrid step bf16 bs=8 max_fetch={max_fetch} frac={frac}")
    dev = G.dev()
    bs = 8
    x = synth.activations(bs, w.H, 0, w.name, step=3).to(dev)
    wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
    oids, ow, _ = oroute.route(G.bits16(x), G.bits16(wg), w.k)
    owner, stamp, clock = synth.foreign_state(w.S, w.E)
    c.set_state(owner, stamp, clock)
    ids = torch.from_numpy(oids).to(dev)
    wts = torch.from_numpy(ow.astype(np.float32)).to(dev)
    slot_ids = torch.empty_like(ids)
    y = torch.empty((bs, w.H), dtype=torch.int16, device=dev)
    ws = torch.empty(c.ffn_workspace_bytes(bs, w.k), dtype=torch.uint8, device=dev)
    c.ensure_experts_hybrid(0, ids, slot_ids, max_fetch, frac)
    c.copy_missing()
    c.expert_ffn(x, slot_ids, wts, y, ws)
    torch.cuda.synchronize()
    c.check()
    t = SlotTable(w.S, w.L, w.E)
    t.set_state(owner, stamp, clock)
    r = t.ensure_hybrid(0, oids, max_fetch, None if frac < 0 else frac)
    assert np.array_equal(slot_ids.cpu().numpy(), r.slot_ids)
    assert c.get_misses() == r.misses
    st = c.stats()
    assert (st["last_indices"], st["last_missing_full"]) == (r.num_indices, r.num_missing_full)
    assert r.num_indices < r.num_missing_full          # the cap bites at this size
    ref = offn.expert_ffn(w.fmt, w.H, w.I, G.bits16(x), r.slot_ids, ow.astype(np.float32).astype(np.float64),
                          lambda s: [hb.row(b, int(t.owner[s]) % w.E).numpy() for b in range(len(hb.banks))])
    err = offn.rel_l2(G.bf16_tensor_to_f64(y), ref)
    print(f"  fetched {r.num_indices} of {r.num_missing_full} misses, rel_l2={err:.3e}")
    assert err <= 1e-2


@pytest.mark.timeout(600)
def test_resize_full_size():
    """Slot-pool resize at the bench workload's size (1024 slots of 9 MiB): shrink to
    300 and grow back; the table matches the oracle and every kept slot keeps its
    bytes (the host row of its layer-0 owner, else the fill)."""
    w, hb, _ = _setup("bf16_h2048")
    _case("resize bf16_h2048 1024 -> 300 -> 1024")
    dev = G.dev()
    sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
    c = oes.Cache(sc, w.S, 0)
    for b, t in enumerate(hb.banks):
        c.set_source(b, 0, t)
    c.fill_slots(0xA5)
    rng = np.random.default_rng(31)
    perm = rng.permutation(w.S)
    owner = np.full(w.S, -1, dtype=np.int64)
    local = perm[: w.E]                                # layer-0 experts, one per slot
    owner[local] = rng.permutation(w.E)
    foreign = perm[w.E: w.E + 500]                     # experts of other layers (no bytes)
    owner[foreign] = w.E + rng.choice((w.L - 1) * w.E, size=500, replace=False)
    stamp = np.where(owner >= 0, rng.integers(1, 400, size=w.S), 0).astype(np.uint64)  # ties on purpose
    c.set_state(owner, stamp, 400)
    c.load_rows(local.tolist(), owner[local].tolist())
    t = SlotTable(w.S, w.L, w.E)
    t.set_state(owner, stamp, 400)

    def check_bytes(carried):
        """Layer-0 owners hold their host rows; other carried-over slots the fill
        (slots past `carried` are new after a grow: their bytes are undefined)."""
        own = t.owner
        loc = np.nonzero((own >= 0) & (own < w.E))[0]
        rest = np.nonzero(~((own >= 0) & (own < w.E)))[0]
        li = torch.from_numpy(loc).to(dev)
        ei = torch.from_numpy(own[loc]).to(dev)
        for b in range(sc.num_banks):
            view = c.slot_bank_view(b)
            rb = hb.row_bytes[b]
            want = hb.banks[b].view(w.E, rb).to(dev)[ei]
            assert torch.equal(view[li], want), b
            kept_fill = [s for s in rest if s < carried]
            if kept_fill:
                assert bool((view[torch.tensor(kept_fill, device=dev)] == 0xA5).all()), b

    t0 = time.perf_counter()
    c.resize(300)
    ms_shrink = (time.perf_counter() - t0) * 1e3
    src = t.resize(300)
    got_owner, got_stamp, clock = c.get_state()
    assert got_owner.tolist() == t.owner.tolist() and got_stamp.tolist() == t.stamp.tolist() and clock == 400
    assert sum(1 for s in src if owner[s] >= 0 and owner[s] < w.E) == int(((t.owner >= 0) & (t.owner < w.E)).sum())
    check_bytes(300)
    t0 = time.perf_counter()
    c.resize(w.S)
    ms_grow = (time.perf_counter() - t0) * 1e3
    t.resize(w.S)
    got_owner, got_stamp, _ = c.get_state()
    assert got_owner.tolist() == t.owner.tolist() and got_stamp.tolist() == t.stamp.tolist()
    check_bytes(300)
    print(f"  shrink {ms_shrink:.1f} ms, grow {ms_grow:.1f} ms", flush=True)
    # a step after the resizes: the remap and the copy agree with the oracle
    ids = synth.synthetic_ids(8, w.k, w.E, 0, w.name).numpy()
    d_ids = torch.from_numpy(ids).to(dev)
    d_slots = torch.empty_like(d_ids)
    c.ensure_experts(0, d_ids, d_slots)
    c.copy_missing()
    torch.cuda.synchronize()
    c.check()
    r = t.ensure(0, ids)
    assert r.status == OK
    assert np.array_equal(d_slots.cpu().numpy(), r.slot_ids)
    assert c.get_misses() == r.misses
    c.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,bs,frac", [("bf16_h2048", 1, 0.5), ("bf16_h2048", 8, 0.3), ("q4_0_h2048", 4, 0.5)])
def test_hybrid_layer_step_full_size(name, bs, frac):
    """The hybrid layer step at full size (every slot foreign, so every routed
    expert misses): fetched experts on the GPU, the rest on the CPU executor;
    y equals the oracle FFN over every routed pair (tokens sampled)."""
    w, hb, c = _setup(name)
    _case(f"hybrid layer step {name} bs={bs} frac={frac}")
    dev = G.dev()
    sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
    cpu = oes.CpuMoe(sc, 0)
    for b, t in enumerate(hb.banks):
        cpu.set_source(b, 0, t)
    x = synth.activations(bs, w.H, 0, w.name, step=11).to(dev)
    wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
    oids, ow, _ = oroute.route(G.bits16(x), G.bits16(wg), w.k)
    ids = torch.from_numpy(oids).to(dev)
    wts = torch.from_numpy(ow.astype(np.float32)).to(dev)
    owner, stamp, clock = synth.foreign_state(w.S, w.E)
    c.set_state(owner, stamp, clock)
    slot_ids = torch.empty_like(ids)
    y = torch.empty((bs, w.H), dtype=torch.int16, device=dev)
    hws, dws = c.hybrid_workspace(bs, w.k)
    host_ws = torch.empty(hws, dtype=torch.uint8, pin_memory=True)
    dev_ws = torch.empty(dws, dtype=torch.uint8, device=dev)
    ffn_ws = torch.empty(c.ffn_workspace_bytes(bs, w.k), dtype=torch.uint8, device=dev)
    c.hybrid_step(cpu, 0, x, ids, wts, slot_ids, y, ffn_ws, host_ws, dev_ws, -1, frac)
    torch.cuda.synchronize()
    c.check()
    t = SlotTable(w.S, w.L, w.E)
    t.set_state(owner, stamp, clock)
    r = t.ensure_hybrid(0, oids, -1, frac)
    assert np.array_equal(slot_ids.cpu().numpy(), r.slot_ids)
    assert len(r.overflow) > 0 and r.num_indices + len(r.overflow) == r.num_missing_full
    sel = [0] if bs == 1 else [0, bs - 1]
    ref = offn.expert_ffn(w.fmt, w.H, w.I, G.bits16(x)[sel], oids[sel], ow[sel].astype(np.float32).astype(np.float64),
                          lambda e: [hb.row(b, int(e)).numpy() for b in range(len(hb.banks))])
    err = offn.rel_l2(G.bf16_tensor_to_f64(y)[sel], ref)
    print(f"  rel_l2={err:.3e} fetched={r.num_indices} cpu={len(r.overflow)}")
    assert err <= (3e-2 if w.fmt in ("nvfp4", "q4_0") else 1e-2)
    cpu.close()
