"""Benchmark arithmetic of the copy benchmark, written out as plain formulas.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FreeToken MoE benchmark guide, §4.3 and §4.4: the flat expert id, the number of
forced misses, the bytes copied, the copy bandwidth and the per-token
extrapolation over all MoE layers.
"""


def flat_id(layer: int, expert: int, num_experts: int) -> int:
    """Flat id of (layer, expert): layer * E + expert (benchmark guide §4.3)."""
    return layer * num_experts + expert


def active_unique(batch: int, topk: int, num_experts: int) -> int:
    """Distinct experts a synthetic step touches: min(E, bs * topk) (§4.3)."""
    return min(num_experts, batch * topk)


def num_misses(active: int, miss_rate: float) -> int:
    """Forced misses: active * miss_rate rounded to an integer (§4.3).

    The page does not say how ties are rounded; Python's round (half to even)
    is taken.  No configuration in use produces an exact .5.
    """
    return int(round(active * miss_rate))


def copy_mib(misses: int, bytes_per_expert: int) -> float:
    """copy_MiB = misses * bytes per expert / 2**20 (§4.4)."""
    return misses * bytes_per_expert / float(1 << 20)


def bw_gbps(misses: int, bytes_per_expert: int, time_ms: float) -> float:
    """Copy bandwidth in GB/s (1e9 B/s) of misses * bytes per expert moved in time_ms (§4.4)."""
    if time_ms <= 0.0:
        raise ValueError("time_ms must be positive")
    return misses * bytes_per_expert / (time_ms * 1.0e6)


def tok_ms(time_ms: float, num_layers: int) -> float:
    """Per-token cost extrapolated over all MoE layers: time_ms * L (§4.4)."""
    return time_ms * num_layers


def decode_tok_s(step_ms: float, num_layers: int) -> float:
    """MoE-layer decode tokens/s at bs=1 when every layer costs step_ms: 1000 / (L * step_ms)."""
    if step_ms <= 0.0:
        raise ValueError("step_ms must be positive")
    return 1000.0 / (num_layers * step_ms)


def hybrid_fetch_fraction(pcie_gbps: float, cpu_gbps: float) -> float:
    """Share of a step's misses a hybrid step fetches over PCIe (FreeToken MoE
    benchmark guide §5.4): overlap is ideal when fetched : CPU-computed experts
    = pcie_bw : (cpu_bw - pcie_bw), i.e. a fetched share of pcie_bw / cpu_bw;
    with a CPU no faster than the link every miss is fetched."""
    if cpu_gbps <= pcie_gbps:
        return 1.0
    return pcie_gbps / cpu_gbps


# Formats whose experts the CPU executor can compute (FreeToken MoE benchmark
# guide §5.2: a format with no CPU MoE weight path - block fp8 is the page's
# example - always stays offload).  Which formats have one is a reading: bf16,
# NVFP4 and GGUF Q4_0 (the decode formats other than block fp8; the MXFP4 banks
# here are the transposed prefill layout).
CPU_FORMATS = ("bf16", "nvfp4", "q4_0")


def recommend_backend(fmt: str, cpu_gbps: float, pcie_gbps: float, threshold: float = 2.0) -> str:
    """ft bench bw's per-(workload, format) decision (benchmark guide §5.2):
    "hybrid" when the CPU MoE kernel's bandwidth exceeds threshold (default 2)
    times the PCIe gather bandwidth and the format has a CPU path, else
    "offload".  Reading: "exceeds" is strict."""
    if fmt not in CPU_FORMATS:
        return "offload"
    return "hybrid" if cpu_gbps > threshold * pcie_gbps else "offload"
