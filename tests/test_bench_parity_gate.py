"""The benchmark's parity gate, on the CPU.

bench.py reports its headline number only when the GPU's headline step (routed
ids, slot map, misses, the bytes copied into the missed slots, the FFN output)
agrees with the oracle's first step.  Here the "GPU step" is the oracle's own
result, fed back in a different miss order, so the gate must pass; each planted
difference (one byte of a slot, a slot id, a routed id, a miss, the FFN output
beyond the tolerance) must make it fail.
"""
import numpy as np
import pytest
import torch

import bench
import synth
from oracle import copy as ocopy
from oracle import ffn as offn
from oracle import route as oroute
from oracle.lru import SlotTable
from synth.workloads import WORKLOADS, make_host_banks

MR = 0.5


@pytest.fixture(scope="module")
def setup():
    w = WORKLOADS["bf16_tiny"]
    hb = make_host_banks(w, device="cpu", pin=False)
    x = synth.activations(1, w.H, 0, w.name)
    wg = synth.router_weight(w.H, w.E, 0, w.name)
    xb = x.numpy().view(np.uint16)
    wgb = wg.numpy().view(np.uint16)
    ids, wts, _ = oroute.route(xb, wgb, w.k)
    active = len(set(ids.ravel().tolist()))
    owner, stamp, clock, _ = synth.forced_miss_state(w.S, w.E, 0, ids, int(round(active * MR)))
    t = SlotTable(w.S, w.L, w.E)
    t.set_state(owner, stamp, clock)
    r = t.ensure(0, ids)
    assert r.misses, "the workload must miss at this rate"
    host = [[hb.banks[b].numpy().reshape(w.E, -1)] for b in range(len(hb.banks))]
    mirror = [np.zeros((w.S, rb), dtype=np.uint8) for rb in hb.row_bytes]
    ocopy.copy_missing(r.misses, host, mirror, w.E)
    y = offn.expert_ffn(w.fmt, w.H, w.I, xb, r.slot_ids, wts,
                        lambda s: [host[b][0][int(t.owner[s]) % w.E] for b in range(len(host))])
    misses = [tuple(m) for m in r.misses][::-1]          # another order than the oracle's
    rows = [m[[sl for sl, _ in misses]].copy() for m in mirror]
    step = {"ids": ids.copy(), "slot_ids": np.array(r.slot_ids).copy(), "y": np.array(y, dtype=np.float64),
            "misses": misses, "rows": rows}
    return w, hb, x, wg, step


def _gate(setup, step):
    w, hb, x, wg, _ = setup
    out = bench._cpu_baseline(w, hb, x, wg, MR, 0.0, step)
    assert out["kind"] == "oracle" and out["value"] > 0
    return out["parity"]


def _copy(step):
    return {k: ([a.copy() for a in v] if k == "rows" else (list(v) if k == "misses" else v.copy()))
            for k, v in step.items()}


def test_gate_passes_on_the_oracle_step(setup):
    p = _gate(setup, setup[4])
    assert p == {"ids": True, "slot_ids": True, "misses": True, "slot_bytes": True,
                 "ffn_rel_l2": 0.0, "ffn_tol": 1e-2, "ok": True}


def test_gate_catches_one_slot_byte(setup):
    s = _copy(setup[4])
    s["rows"][1][0, 7] ^= 1
    p = _gate(setup, s)
    assert p["misses"] and not p["slot_bytes"] and not p["ok"]


def test_gate_catches_slot_map_and_ids(setup):
    s = _copy(setup[4])
    s["slot_ids"].flat[0] = (s["slot_ids"].flat[0] + 1) % setup[0].S
    p = _gate(setup, s)
    assert not p["slot_ids"] and p["ids"] and not p["ok"]
    s = _copy(setup[4])
    s["ids"].flat[0] = (s["ids"].flat[0] + 1) % setup[0].E
    p = _gate(setup, s)
    assert not p["ids"] and not p["ok"]


def test_gate_catches_a_wrong_miss(setup):
    s = _copy(setup[4])
    sl, e = s["misses"][0]
    s["misses"][0] = (sl, e + 1)
    p = _gate(setup, s)
    assert not p["misses"] and not p["slot_bytes"] and not p["ok"]


def test_gate_ffn_tolerance(setup):
    s = _copy(setup[4])
    s["y"] = s["y"] * (1 + 0.5e-2)                       # within 1e-2
    p = _gate(setup, s)
    assert p["ok"] and 0 < p["ffn_rel_l2"] <= 1e-2
    s["y"] = setup[4]["y"] * (1 + 2e-2)                  # beyond it
    p = _gate(setup, s)
    assert not p["ok"] and p["ffn_rel_l2"] > 1e-2
