"""The decode FFN's grouped path (several tokens: pairs grouped by slot, each
expert's rows read once and dotted with every token routed to it; selected with
OES_OPT_FFN_PATH) against the oracle, on the cases the grouping itself creates: one expert taking every token
(groups longer than one LDS pass, down to passes of two rows at a wide H), an
out-of-range slot (reported, its pair left out), a pool of 4096 slots, and many
tokens over few experts."""
import numpy as np
import pytest
import torch

import offloaded_expert_slot_amd as oes
import synth
from oracle import ffn as offn
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _run(fmt, H, I, E, S, slot_ids, tag, rows_of_slot, host, bad=None):
    n, k = slot_ids.shape
    c = G.make_cache(fmt, 1, E, H, I, S, {0: host})
    c.set_option(oes.OPT_FFN_PATH, oes.FFN_GROUPED)
    c.load_rows(list(rows_of_slot.keys()), list(rows_of_slot.values()))
    rng = np.random.default_rng(n * 7 + k)
    w = rng.random((n, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    x = synth.activations(n, H, 0, tag).to(G.dev())
    d_slots = torch.from_numpy(slot_ids).to(G.dev())
    y = torch.full((n, H), 0x7fff, dtype=torch.int16, device=G.dev())
    ws = torch.empty(c.ffn_workspace_bytes(n, k), dtype=torch.uint8, device=G.dev())
    c.expert_ffn(x, d_slots, torch.from_numpy(w).to(G.dev()), y, ws)
    torch.cuda.synchronize()
    if bad is None:
        c.check()
    else:
        assert c.check_status() == oes.ERR_ARG
    used = np.where((slot_ids >= 0) & (slot_ids < S), slot_ids, -1)
    hb = G.oracle_host({0: host}, 1, len(host.banks))
    ref = offn.expert_ffn(fmt, H, I, G.bits16(x), used, w.astype(np.float64),
                          lambda s: [hb[b][0][rows_of_slot[int(s)]] for b in range(len(hb))])
    got = G.bf16_tensor_to_f64(y)
    err = offn.rel_l2(got, ref)
    worst = max(offn.rel_l2(got[i:i + 1], ref[i:i + 1]) for i in range(n))
    print(f"  rel_l2={err:.3e} worst token {worst:.3e}")
    assert err <= 5e-3 and worst <= (1e-2 if fmt == "bf16" else 3e-2)
    c.close()


@pytest.mark.parametrize("fmt,H,I", [("bf16", 512, 256), ("nvfp4", 7168, 256), ("q4_0", 4096, 512),
                                     ("fp8_block128", 1024, 256)])
def test_hot_expert_longer_than_a_pass(fmt, H, I):
    """Every token routes to slot 3 (a group of 21 pairs: several LDS passes), the
    other pair of each token to one of a few slots."""
    E, k, n = 8, 2, 21
    _case(f"grouped ffn hot expert {fmt} H={H} I={I} n={n}")
    host = G.make_banks(fmt, E, H, I, tag=f"grp-{fmt}")
    rng = np.random.default_rng(5)
    slot_ids = np.stack([[3, int(rng.choice([0, 1, 5, 6]))] for _ in range(n)]).astype(np.int32)
    slot_ids[4, 1] = -1                       # a skipped pair
    _run(fmt, H, I, E, E, slot_ids, f"grp-{fmt}", {s: (s * 3 + 2) % E for s in range(E)}, host)


def test_out_of_range_slot_is_reported_and_left_out():
    fmt, H, I, E, k, n = "bf16", 512, 256, 8, 3, 6
    _case("grouped ffn slot past the pool")
    host = G.make_banks(fmt, E, H, I, tag="grp-bad")
    rng = np.random.default_rng(9)
    slot_ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    slot_ids[2, 1] = E + 5                    # past the pool: reported, the pair left out
    _run(fmt, H, I, E, E, slot_ids, "grp-bad", {s: s for s in range(E)}, host, bad=True)


def test_large_pool_and_many_tokens():
    """4096 slots (the grouping's slot histogram at its limit), 96 tokens top-8 over
    40 experts held in scattered slots."""
    fmt, H, I, E, k, n, S = "bf16", 256, 128, 40, 8, 96, 4096
    _case(f"grouped ffn S={S} n={n} k={k}")
    host = G.make_banks(fmt, E, H, I, tag="grp-big")
    rng = np.random.default_rng(11)
    slots = rng.choice(S, size=E, replace=False)          # expert e lives in slot slots[e]
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)])
    slot_ids = slots[ids].astype(np.int32)
    _run(fmt, H, I, E, S, slot_ids, "grp-big", {int(slots[e]): e for e in range(E)}, host)
