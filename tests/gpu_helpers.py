"""Shared setup of the GPU parity tests (not a test module)."""
import numpy as np
import torch

import offloaded_expert_slot_amd as oes
import synth
from synth.workloads import HostBanks, Workload, make_host_banks


def dev():
    return torch.device("cuda:0")


def make_banks(fmt, E, H, I, layer=0, tag="t", seed=0):
    w = Workload(tag, fmt, L=layer + 1, E=E, k=1, H=H, I=I, S=1)
    return make_host_banks(w, layer=layer, seed=seed)


def make_cache(fmt, L, E, H, I, S, banks_by_layer):
    """Cache with `banks_by_layer[layer] = HostBanks` registered as sources."""
    sc = oes.schema_make(fmt, L, E, H, I)
    c = oes.Cache(sc, S, 0)
    for layer, hb in banks_by_layer.items():
        assert hb.row_bytes == sc.row_bytes()
        for b, t in enumerate(hb.banks):
            c.set_source(b, layer, t)
    return c


def oracle_host(banks_by_layer, L, num_banks):
    """host_banks[b][layer] numpy [E, row_bytes] views for the oracle (None where absent)."""
    out = []
    for b in range(num_banks):
        per = []
        for layer in range(L):
            hb = banks_by_layer.get(layer)
            per.append(None if hb is None else hb.banks[b].numpy().reshape(hb.E, hb.row_bytes[b]))
        out.append(per)
    return out


def slot_bytes(cache, bank):
    """Copy of slot bank `bank` as numpy uint8 [S, row_bytes]."""
    return cache.slot_bank_view(bank).cpu().numpy()


def bits16(t):
    """int16 torch tensor of bf16 bits -> numpy uint16."""
    return t.cpu().numpy().view(np.uint16)


def bf16_tensor_to_f64(t):
    return t.view(torch.bfloat16).double().cpu().numpy()
