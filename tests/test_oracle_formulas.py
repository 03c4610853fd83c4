"""Pins of the benchmark arithmetic and of the bank schemas.

The expected numbers are worked by hand from the formulas stated in the
FreeToken MoE benchmark guide (§4.3: flat id, active = min(E, bs*topk),
misses = active * miss_rate rounded; §4.4: copy_MiB = misses * bytes per
expert, tok_ms = time_ms * L) and from the configuration sizes; they are typed
in here, not recomputed with the oracle's code.
"""
import pytest

from oracle import formulas as F
from oracle import schema


def test_flat_id():
    assert F.flat_id(0, 5, 128) == 5
    assert F.flat_id(3, 7, 16) == 55
    assert F.flat_id(59, 255, 256) == 15359


@pytest.mark.parametrize("E,bs,k,mr,active,misses", [
    (16, 1, 2, 0.5, 2, 1), (16, 4, 2, 0.5, 8, 4),
    (128, 1, 8, 0.0, 8, 0), (128, 1, 8, 0.25, 8, 2), (128, 1, 8, 0.5, 8, 4), (128, 1, 8, 1.0, 8, 8),
    (128, 8, 8, 0.25, 64, 16), (128, 8, 8, 0.5, 64, 32), (128, 8, 8, 1.0, 64, 64),
    (128, 32, 8, 0.25, 128, 32), (128, 32, 8, 0.5, 128, 64), (128, 32, 8, 1.0, 128, 128),
    (256, 1, 8, 0.1, 8, 1), (256, 1, 8, 0.5, 8, 4), (256, 16, 8, 0.1, 128, 13), (256, 16, 8, 0.5, 128, 64),
    (256, 1, 8, 0.05, 8, 0), (256, 1, 8, 0.25, 8, 2), (256, 1, 8, 1.0, 8, 8),
    (256, 4, 8, 0.05, 32, 2), (256, 4, 8, 0.25, 32, 8), (256, 4, 8, 1.0, 32, 32),
])
def test_active_and_misses(E, bs, k, mr, active, misses):
    a = F.active_unique(bs, k, E)
    assert a == active
    assert F.num_misses(a, mr) == misses


def test_round_half_even_reading():
    # the page says "rounded"; half-to-even is the reading taken
    assert F.num_misses(5, 0.5) == 2
    assert F.num_misses(3, 0.5) == 2


@pytest.mark.parametrize("fmt,H,I,bpe,banks", [
    ("bf16", 256, 128, 196608, [131072, 65536]),
    ("bf16", 2048, 768, 9437184, [6291456, 3145728]),
    ("fp8_block128", 4096, 1536, 18878976, [12582912, 3072, 6291456, 1536]),
    ("nvfp4", 7168, 2048, 24795136, [14680064, 1835008, 8192, 7340032, 917504, 14336]),
    ("mxfp4_t", 2880, 2880, 13236480, [8294400, 518400, 11520, 4147200, 259200, 5760]),
    ("q4_0", 2048, 768, 2654208, [1572864, 196608, 786432, 98304]),
])
def test_bank_bytes(fmt, H, I, bpe, banks):
    specs = schema.bank_specs(fmt, H, I)
    assert [s[3] for s in specs] == banks
    assert schema.bytes_per_expert(fmt, H, I) == bpe


def test_copy_mib_and_tok_ms():
    assert F.copy_mib(16, 9437184) == pytest.approx(144.0)
    assert F.copy_mib(13, 18878976) == pytest.approx(234.0572, abs=1e-3)
    assert F.copy_mib(32, 24795136) == pytest.approx(756.6875, abs=1e-4)
    assert F.tok_ms(0.5, 48) == pytest.approx(24.0)
    # 72 MiB in 1.5 ms is 75497472 B / 1.5e-3 s = 50.33 GB/s
    assert F.bw_gbps(8, 9437184, 1.5) == pytest.approx(50.331648)
    assert F.decode_tok_s(0.25, 48) == pytest.approx(1000.0 / 12.0)
    with pytest.raises(ValueError):
        F.bw_gbps(1, 1, 0.0)


def test_recommend_backend_closed_forms():
    """Benchmark guide §5.2: hybrid iff the CPU kernel beats threshold x the PCIe gather,
    and only for formats with a CPU path."""
    assert F.recommend_backend("bf16", 120.0, 56.0) == "hybrid"      # 120 > 2 * 56
    assert F.recommend_backend("bf16", 112.0, 56.0) == "offload"     # equal: not exceeding
    assert F.recommend_backend("bf16", 100.0, 56.0) == "offload"
    assert F.recommend_backend("nvfp4", 100.0, 40.0, threshold=2.5) == "offload"
    assert F.recommend_backend("nvfp4", 100.1, 40.0, threshold=2.5) == "hybrid"
    assert F.recommend_backend("q4_0", 57.0, 56.0, threshold=1.0) == "hybrid"
    assert F.recommend_backend("fp8_block128", 1e6, 1.0) == "offload"
    assert F.recommend_backend("mxfp4_t", 1e6, 1.0) == "offload"
    assert set(F.CPU_FORMATS) == {"bf16", "nvfp4", "q4_0"}
