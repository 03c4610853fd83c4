"""The six synthetic workloads and builders for their host banks.

Sizes follow the workloads the benchmark is quoted on; inputs are seeded
(seed 0) and synthetic.  Only layer 0's host banks are filled, as the copy
benchmark of the FreeToken MoE benchmark guide (§4.4) drives layer 0 only;
the other layers' sources stay unregistered.

This module only allocates and fills input memory; it computes nothing of the
step itself.
"""
from dataclasses import dataclass, field

import torch

from . import expert_rows, fill_layer_banks


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str
    L: int
    E: int
    k: int
    H: int
    I: int
    S: int
    batches: tuple = ()
    miss_rates: tuple = ()
    tokens: int = 0          # prefill tokens
    stream_layers: int = 0   # prefill layers streamed through the double buffer
    note: str = ""


WORKLOADS = {
    w.name: w for w in [
        Workload("bf16_tiny", "bf16", L=1, E=16, k=2, H=256, I=128, S=8, batches=(1, 4), miss_rates=(0.5,),
                 note="tiny bf16 parity workload, 8 slots owned by a foreign layer"),
        Workload("bf16_h2048", "bf16", L=48, E=128, k=8, H=2048, I=768, S=1024, batches=(1, 8, 32),
                 miss_rates=(0.0, 0.25, 0.5, 1.0), note="bf16 decode sweep, 48 layers, 1024 slots"),
        Workload("fp8_h4096", "fp8_block128", L=60, E=256, k=8, H=4096, I=1536, S=2048, batches=(1, 16),
                 miss_rates=(0.1, 0.5), note="fp8 128x128-block banks, 60 layers, 2048 slots"),
        Workload("nvfp4_h7168", "nvfp4", L=60, E=256, k=8, H=7168, I=2048, S=1536, batches=(1, 4),
                 miss_rates=(0.05, 0.25, 1.0), note="nvfp4 six-bank layout, 60 layers, 1536 slots"),
        Workload("q4_0_h2048", "q4_0", L=48, E=128, k=8, H=2048, I=768, S=1024, batches=(1, 8),
                 miss_rates=(0.25, 0.5), note="GGUF Q4_0 banks at the bf16 sweep's model shape, 1024 slots"),
        Workload("mxfp4_prefill", "mxfp4_t", L=4, E=128, k=4, H=2880, I=2880, S=0, tokens=2048,
                 stream_layers=4, note="mxfp4 transposed banks streamed per layer, 2048 tokens"),
    ]
}


def bank_row_bytes(fmt, hidden, inter):
    """Row bytes per bank, measured from one generated expert."""
    return [r.numel() for r in expert_rows(fmt, hidden, inter, 0, "size-probe", 0, "cpu")]


@dataclass
class HostBanks:
    """Pinned host banks of one layer: banks[b] is uint8 [E * row_bytes_b]."""
    fmt: str
    E: int
    row_bytes: list
    banks: list = field(default_factory=list)

    def row(self, b, e):
        rb = self.row_bytes[b]
        return self.banks[b][e * rb:(e + 1) * rb]

    def expert_rows(self, e):
        return [self.row(b, e) for b in range(len(self.banks))]


def make_host_banks(w: Workload, layer=0, seed=0, device=None, pin=True):
    """Allocate pinned host banks for `layer` of workload `w` and fill them with seeded experts.

    Expert rows are drawn on `device` (CUDA when available: much faster) and
    copied into the pinned banks.
    """
    if device is None:
        device = "cuda" if torch.cuda.is_available() else "cpu"
    rbs = bank_row_bytes(w.fmt, w.H, w.I)
    banks = [torch.empty(w.E * rb, dtype=torch.uint8, pin_memory=pin) for rb in rbs]
    fill_layer_banks(w.fmt, w.H, w.I, w.E, layer, seed, w.name, banks, device)
    if device != "cpu":
        torch.cuda.synchronize()
    return HostBanks(w.fmt, w.E, rbs, banks)
