"""Hybrid backend on the GPU machine: the CPU MoE executor (host cores) and the
whole hybrid layer step (GPU remap, copy and FFN; CPU executor for the -1
experts; combine), against the oracle.

The executor's reference is the oracle FFN over the pairs it takes; the hybrid
step's is the oracle FFN over every routed pair - splitting the experts between
GPU and CPU must not change the result beyond rounding - and the oracle's
ensure_experts_hybrid for the slot map and the table.
"""
import numpy as np
import pytest
import torch

import offloaded_expert_slot_amd as oes
import synth
from oracle import ffn as offn
from oracle.lru import OK, SlotTable
from synth.workloads import Workload, make_host_banks
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _tol(fmt):
    return 3e-2 if fmt in ("nvfp4", "q4_0") else 1e-2


def _banks(fmt, E, H, I, layer=0, tag="hy"):
    return make_host_banks(Workload(tag, fmt, L=layer + 1, E=E, k=1, H=H, I=I, S=1), layer=layer)


def _rows(hb):
    return lambda e: [hb.row(b, int(e)).numpy() for b in range(len(hb.banks))]


# ------------------------------------------------------------------ the executor
@pytest.mark.parametrize("fmt,H,I,E,n,k", [
    ("bf16", 256, 128, 8, 3, 4), ("nvfp4", 512, 256, 8, 3, 4), ("q4_0", 512, 256, 8, 3, 4),
    ("bf16", 2048, 768, 16, 1, 8), ("q4_0", 2048, 768, 16, 4, 8), ("nvfp4", 7168, 2048, 6, 2, 4),
    ("bf16", 264, 136, 5, 2, 3),   # K not a multiple of 32: the masked tail
    ("nvfp4", 288, 160, 6, 2, 3),  # rows not a multiple of 64: element-order nvfp4 path
    ("nvfp4", 512, 160, 6, 2, 3),  # even/odd path for gate_up, element order for down
    ("nvfp4", 4160, 192, 5, 1, 4), # 65 64-element steps: scales masked at the row's end
])
def test_cpu_moe_matches_oracle(fmt, H, I, E, n, k):
    _case(f"cpu moe {fmt} H={H} I={I} n={n} k={k}")
    hb = _banks(fmt, E, H, I, tag=f"cpu-{fmt}-{H}")
    sc = oes.schema_make(fmt, 1, E, H, I)
    rng = np.random.default_rng(H + n)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    slots = np.where(rng.random((n, k)) < 0.6, -1, 3).astype(np.int32)
    slots[0, 0] = -1
    w = rng.random((n, k)).astype(np.float32)
    x = synth.activations(n, H, 0, f"cpu-{fmt}")
    ys = []
    for threads in (1, 3, 0):
        m = oes.CpuMoe(sc, threads)
        for b, t in enumerate(hb.banks):
            m.set_source(b, 0, t)
        y = np.full((n, H), np.nan, dtype=np.float32)
        m.run(0, x, ids, slots, w, y)
        ys.append(y)
        m.close()
    # the summation order does not depend on the thread count
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
    ref = offn.expert_ffn(fmt, H, I, x.numpy().view(np.uint16), np.where(slots < 0, ids, -1),
                          w.astype(np.float64), _rows(hb))
    err = offn.rel_l2(ys[0].astype(np.float64), ref)
    print(f"  rel_l2={err:.3e}")
    assert err <= _tol(fmt) and err <= 5e-3
    # tokens with no CPU pair get zeros
    none = np.nonzero((slots >= 0).all(axis=1))[0]
    assert (ys[0][none] == 0).all()


def test_cpu_moe_errors():
    _case("cpu moe errors")
    for fmt in ("fp8_block128", "mxfp4_t"):
        with pytest.raises(oes.OesError) as ei:
            oes.CpuMoe(oes.schema_make(fmt, 1, 4, 256, 256))
        assert ei.value.status == oes.ERR_UNSUPPORTED
    sc = oes.schema_make("bf16", 2, 4, 64, 64)
    m = oes.CpuMoe(sc, 2)
    hb = _banks("bf16", 4, 64, 64, tag="cpu-err")
    for b, t in enumerate(hb.banks):
        m.set_source(b, 0, t)
    x = torch.zeros((1, 64), dtype=torch.int16)
    y = np.zeros((1, 64), dtype=np.float32)
    w = np.ones((1, 2), dtype=np.float32)
    with pytest.raises(oes.OesError) as ei:                       # an id outside [0, E)
        m.run(0, x, np.array([[1, 4]], np.int32), np.array([[-1, -1]], np.int32), w, y)
    assert ei.value.status == oes.ERR_ARG
    with pytest.raises(oes.OesError) as ei:                       # layer 1 has no source
        m.run(1, x, np.array([[1, 2]], np.int32), np.array([[-1, 0]], np.int32), w, y)
    assert ei.value.status == oes.ERR_ARG
    m.run(1, x, np.array([[1, 2]], np.int32), np.array([[5, 0]], np.int32), w, y)  # no CPU pair: fine
    assert (y == 0).all()
    with pytest.raises(oes.OesError):
        m.set_source(0, 0, hb.banks[0][:-16])                    # wrong size


# ------------------------------------------------------------------ the hybrid step
def _hybrid(fmt, H, I, E, S, L, layer, n, k, steps, max_fetch, frac, seed):
    banks = {layer: _banks(fmt, E, H, I, layer=layer, tag=f"hy-{fmt}")}
    c = G.make_cache(fmt, L, E, H, I, S, banks)
    sc = oes.schema_make(fmt, L, E, H, I)
    cpu = oes.CpuMoe(sc, 0)
    for b, t in enumerate(banks[layer].banks):
        cpu.set_source(b, layer, t)
    t = SlotTable(S, L, E)
    hb = banks[layer]
    dev = G.dev()
    rng = np.random.default_rng(seed)
    hws, dws = c.hybrid_workspace(n, k)
    host_ws = torch.empty(hws, dtype=torch.uint8, pin_memory=True)
    dev_ws = torch.empty(dws, dtype=torch.uint8, device=dev)
    ffn_ws = torch.empty(c.ffn_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    for step in range(steps):
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)]).astype(np.int32)
        w = rng.random((n, k)).astype(np.float32)
        w /= w.sum(axis=1, keepdims=True)
        x = synth.activations(n, H, 0, f"hy-{fmt}", step=step).to(dev)
        d_ids, d_w = torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
        d_slots = torch.empty_like(d_ids)
        y = torch.empty((n, H), dtype=torch.int16, device=dev)
        c.hybrid_step(cpu, layer, x, d_ids, d_w, d_slots, y, ffn_ws, host_ws, dev_ws, max_fetch, frac)
        torch.cuda.synchronize()
        c.check()
        r = t.ensure_hybrid(layer, ids, max_fetch, None if frac < 0 else frac)
        assert r.status == OK
        assert np.array_equal(d_slots.cpu().numpy(), r.slot_ids), step
        owner, stamp, clock = c.get_state()
        assert owner.tolist() == t.owner.tolist() and stamp.tolist() == t.stamp.tolist() and clock == t.clock
        # the split does not change y: the oracle FFN over every routed pair
        ref = offn.expert_ffn(fmt, H, I, G.bits16(x), ids, w.astype(np.float64), _rows(hb))
        err = offn.rel_l2(G.bf16_tensor_to_f64(y), ref)
        assert err <= _tol(fmt) and err <= 5e-3, (step, err)
        yield r
    cpu.close()
    c.close()


@pytest.mark.parametrize("fmt,H,I", [("bf16", 256, 128), ("nvfp4", 512, 256), ("q4_0", 512, 256)])
@pytest.mark.parametrize("max_fetch,frac", [(1, -1.0), (-1, 0.5), (0, -1.0)])
def test_hybrid_step_matches_oracle(fmt, H, I, max_fetch, frac):
    _case(f"hybrid step {fmt} max_fetch={max_fetch} frac={frac}")
    cpu_pairs = 0
    for r in _hybrid(fmt, H, I, E=12, S=6, L=2, layer=1, n=3, k=3, steps=6, max_fetch=max_fetch, frac=frac,
                     seed=7):
        cpu_pairs += len(r.overflow)
    assert cpu_pairs > 0          # the CPU executor took part


def test_hybrid_step_all_fetched():
    """A cap at or above the misses: no -1 pair, the step equals the plain one."""
    _case("hybrid step, every miss fetched")
    for r in _hybrid("bf16", 256, 128, E=8, S=8, L=1, layer=0, n=2, k=2, steps=4, max_fetch=99, frac=-1.0,
                     seed=3):
        assert r.overflow == []
