"""The benchmark's parity gate, on the CPU.

bench.py checks every measured row's step against the oracle's step on the same
inputs (routed ids, slot map, the miss list in install order, the bytes copied
into the missed slots of every bank, the FFN output) and reports a row's numbers
as valid only when they agree.  Here the "GPU step" is the oracle's own result fed
back in, so the gate must pass; each planted difference (one byte of a slot, a
slot id, a routed id, a miss, the miss order, the FFN output beyond the tolerance)
must make it fail.
"""
import numpy as np
import pytest

import bench
import synth
from oracle import formulas
from oracle import route as oroute
from synth.workloads import WORKLOADS, make_host_banks

MR = 0.5


@pytest.fixture(scope="module")
def setup():
    w = WORKLOADS["bf16_tiny"]
    n = 4
    hb = make_host_banks(w, device="cpu", pin=False)
    xb = synth.activations(n, w.H, 0, w.name).numpy().view(np.uint16)
    wgb = synth.router_weight(w.H, w.E, 0, w.name).numpy().view(np.uint16)
    ids, _, _ = oroute.route(xb, wgb, w.k)
    active = len(set(ids.ravel().tolist()))
    owner, stamp, clock, _ = synth.forced_miss_state(w.S, w.E, 0, ids, formulas.num_misses(active, MR))
    host = [[hb.banks[b].numpy().reshape(w.E, -1)] for b in range(len(hb.banks))]
    step, times = bench._oracle_step(w, host, (owner, stamp, clock), hb.row_bytes, xb=xb, wgb=wgb)
    assert len(step["misses"]) >= 2, "the workload must miss more than once at this rate"
    assert set(times) == {"t_route_ms", "t_ensure_ms", "t_copy_ms", "t_ffn_ms", "ms_per_step"}
    return w, step


def _copy(step):
    return {k: ([a.copy() for a in v] if k == "rows" else (list(v) if k == "misses" else
                                                           (None if v is None else np.copy(v))))
            for k, v in step.items()}


def test_gate_passes_on_the_oracle_step(setup):
    w, step = setup
    p = bench._gate(_copy(step), step, bench._tol(w.fmt))
    assert p == {"ids": True, "slot_ids": True, "misses": True, "slot_bytes": True,
                 "ffn_rel_l2": 0.0, "ffn_tol": 1e-2, "ok": True}


def test_gate_catches_one_slot_byte(setup):
    w, step = setup
    s = _copy(step)
    s["rows"][1][0, 7] ^= 1
    p = bench._gate(s, step, 1e-2)
    assert p["misses"] and not p["slot_bytes"] and not p["ok"]


def test_gate_catches_slot_map_and_ids(setup):
    w, step = setup
    s = _copy(step)
    s["slot_ids"].flat[0] = (s["slot_ids"].flat[0] + 1) % w.S
    p = bench._gate(s, step, 1e-2)
    assert not p["slot_ids"] and p["ids"] and not p["ok"]
    s = _copy(step)
    s["ids"].flat[0] = (s["ids"].flat[0] + 1) % w.E
    p = bench._gate(s, step, 1e-2)
    assert not p["ids"] and not p["ok"]


def test_gate_catches_a_wrong_miss_and_the_miss_order(setup):
    w, step = setup
    s = _copy(step)
    sl, e = s["misses"][0]
    s["misses"][0] = (sl, e + 1)
    p = bench._gate(s, step, 1e-2)
    assert not p["misses"] and not p["slot_bytes"] and not p["ok"]
    s = _copy(step)
    s["misses"] = s["misses"][::-1]
    s["rows"] = [r[::-1].copy() for r in s["rows"]]
    p = bench._gate(s, step, 1e-2)
    assert not p["misses"] and not p["ok"]


def test_gate_ffn_tolerance(setup):
    w, step = setup
    s = _copy(step)
    s["y"] = step["y"] * (1 + 0.5e-2)                    # within 1e-2
    p = bench._gate(s, step, 1e-2)
    assert p["ok"] and 0 < p["ffn_rel_l2"] <= 1e-2
    s["y"] = step["y"] * (1 + 2e-2)                      # beyond it
    p = bench._gate(s, step, 1e-2)
    assert not p["ok"] and p["ffn_rel_l2"] > 1e-2


def test_copy_row_gate_without_ffn(setup):
    """Copy-sweep rows are gated on the remap and the bytes only."""
    w, _ = setup
    hb = make_host_banks(w, device="cpu", pin=False)
    host = [[hb.banks[b].numpy().reshape(w.E, -1)] for b in range(len(hb.banks))]
    sids = synth.synthetic_ids(4, w.k, w.E, 0, w.name).numpy()
    m = formulas.num_misses(formulas.active_unique(4, w.k, w.E), MR)
    owner, stamp, clock, _ = synth.forced_miss_state(w.S, w.E, 0, sids, m)
    step, times = bench._oracle_step(w, host, (owner, stamp, clock), hb.row_bytes, ids=sids, ffn=False)
    assert len(step["misses"]) == m and step["y"] is None and "t_ffn_ms" not in times
    p = bench._gate(_copy(step), step, routed=False)
    assert p == {"slot_ids": True, "misses": True, "slot_bytes": True, "ok": True}
