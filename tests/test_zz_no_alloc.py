"""oes_expert_ffn_noalloc (the FFN on the library's own per-GPU scratch array) against
oes_expert_ffn with a caller workspace: the same kernels, so the outputs must be
bit-identical.  Two calls in a row on one cache, the second with fewer tokens, so a
stale scratch from the first call would show; a size beyond the array is refused
before any GPU work."""
import numpy as np
import pytest
import torch

import offloaded_expert_slot_amd as oes
import synth
from oracle import ffn as offn
from oracle.lru import SlotTable
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("path", ["per_pair", "grouped"])
@pytest.mark.parametrize("fmt,H,I,E,k", [("bf16", 256, 128, 16, 2), ("fp8_block128", 1024, 512, 16, 4),
                                         ("nvfp4", 512, 256, 16, 4), ("q4_0", 512, 256, 16, 8)])
def test_noalloc_matches_workspace_entry_point(fmt, H, I, E, k, path):
    dev = G.dev()
    hb = G.make_banks(fmt, E, H, I, tag=f"na-{fmt}")
    S = E
    c = G.make_cache(fmt, 1, E, H, I, S, {0: hb})
    c.set_option(oes.OPT_FFN_PATH, oes.FFN_GROUPED if path == "grouped" else oes.FFN_PER_PAIR)
    owner, stamp, clock = synth.foreign_state(S, E)
    for n in (16, 3):   # the second call is smaller
        _case(f"noalloc {fmt} H={H} I={I} E={E} k={k} n={n} path={path}")
        c.set_state(owner, stamp, clock)
        rng = np.random.default_rng(n)
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)]).astype(np.int32)
        wts = rng.random((n, k)).astype(np.float32)
        wts /= wts.sum(axis=1, keepdims=True)
        x = synth.activations(n, H, 0, f"na-{fmt}", step=n).to(dev)
        d_ids = torch.from_numpy(ids).to(dev)
        d_w = torch.from_numpy(wts).to(dev)
        slot_ids = torch.empty_like(d_ids)
        c.ensure_experts(0, d_ids, slot_ids)
        c.copy_missing()
        y_ref = torch.full((n, H), 0x7fff, dtype=torch.int16, device=dev)
        y_na = torch.full((n, H), 0x7fff, dtype=torch.int16, device=dev)
        ws = torch.empty(c.ffn_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
        c.expert_ffn(x, slot_ids, d_w, y_ref, ws)
        c.expert_ffn_noalloc(x, slot_ids, d_w, y_na)
        torch.cuda.synchronize()
        c.check()
        assert torch.equal(y_na, y_ref)
        # and both are the oracle's FFN within the format's tolerance
        t = SlotTable(S, 1, E)
        t.set_state(owner, stamp, clock)
        r = t.ensure(0, ids)
        assert np.array_equal(slot_ids.cpu().numpy(), r.slot_ids)
        ref = offn.expert_ffn(fmt, H, I, G.bits16(x), r.slot_ids, wts.astype(np.float64),
                              lambda s: [hb.row(b, int(t.owner[s]) % E).numpy() for b in range(len(hb.banks))])
        err = offn.rel_l2(G.bf16_tensor_to_f64(y_na), ref)
        print(f"  rel_l2={err:.3e}")
        assert err <= (3e-2 if fmt in ("nvfp4", "q4_0") else 1e-2)
    c.close()


def _largest_n(c, k):
    """The most tokens whose workspace fits the scratch array (host-side sizes only)."""
    lo, hi = 1, 32768 // k
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if c.ffn_workspace_bytes(mid, k) <= oes.FFN_NOALLOC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid - 1
    return lo


def test_noalloc_at_the_limit_and_beyond():
    """The largest call the array holds matches the workspace entry point; one token
    more is refused before any GPU work."""
    dev = G.dev()
    fmt, H, I, E, k = "bf16", 256, 128, 16, 2
    hb = G.make_banks(fmt, E, H, I, tag="na-limit")
    c = G.make_cache(fmt, 1, E, H, I, E, {0: hb})
    c.set_option(oes.OPT_FFN_PATH, oes.FFN_GROUPED)    # the larger workspace of the two paths
    c.load_rows(list(range(E)), list(range(E)))
    n_ok = _largest_n(c, k)
    n = n_ok + 1
    _case(f"noalloc limit n_ok={n_ok}")
    assert c.ffn_workspace_bytes(n_ok, k) <= oes.FFN_NOALLOC_SCRATCH_BYTES < c.ffn_workspace_bytes(n, k)
    rng = np.random.default_rng(2)
    slot_ids = torch.from_numpy(rng.integers(0, E, size=(n, k)).astype(np.int32)).to(dev)
    w = torch.full((n, k), 0.5, dtype=torch.float32, device=dev)
    x = synth.activations(n, H, 0, "na-limit").to(dev)
    y = torch.full((n, H), 7, dtype=torch.int16, device=dev)
    with pytest.raises(oes.OesError) as ei:
        c.expert_ffn_noalloc(x, slot_ids, w, y)
    assert ei.value.status == oes.ERR_ARG and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((y == 7).all())          # nothing was enqueued
    y_na = torch.empty((n_ok, H), dtype=torch.int16, device=dev)
    y_ref = torch.empty_like(y_na)
    ws = torch.empty(c.ffn_workspace_bytes(n_ok, k), dtype=torch.uint8, device=dev)
    c.expert_ffn(x[:n_ok], slot_ids[:n_ok], w[:n_ok], y_ref, ws)
    c.expert_ffn_noalloc(x[:n_ok], slot_ids[:n_ok], w[:n_ok], y_na)
    torch.cuda.synchronize()
    c.check()
    assert torch.equal(y_na, y_ref)
    c.close()
