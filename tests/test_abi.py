"""CPU checks of the C ABI: the library loads, exports every declared function,
and rejects bad arguments before touching a GPU.  No compute call is made."""
import ctypes

import numpy as np
import pytest

import offloaded_expert_slot_amd as oes
from oracle import schema as oschema


@pytest.fixture(scope="module")
def L():
    return oes.lib()


def test_exports_every_declared_symbol(L):
    names = oes.header_functions()
    assert len(names) >= 30
    for n in names:
        assert hasattr(L, n), n
        assert n in oes._SIGS, f"binding lacks {n}"


def test_status_strings_and_version(L):
    assert L.oes_abi_version() == 1
    assert L.oes_status_str(0) == b"OES_OK"
    assert L.oes_status_str(-2) == b"OES_ERR_CAPACITY"
    assert L.oes_status_str(-99) == b"OES_ERR_UNKNOWN"


@pytest.mark.parametrize("fmt,H,I", [("bf16", 256, 128), ("bf16", 2048, 768), ("fp8_block128", 4096, 1536),
                                     ("nvfp4", 7168, 2048), ("mxfp4_t", 2880, 2880)])
def test_schema_matches_oracle(fmt, H, I):
    sc = oes.schema_make(fmt, 3, 16, H, I)
    specs = oschema.bank_specs(fmt, H, I)
    assert sc.bank_names() == [s[0] for s in specs]
    assert sc.row_bytes() == [s[3] for s in specs]
    assert sc.bytes_per_expert == oschema.bytes_per_expert(fmt, H, I)


@pytest.mark.parametrize("args", [
    (0, 0, 16, 256, 128), (0, 1, 0, 256, 128), (0, 1, 16, 250, 128), (1, 1, 16, 200, 128),
    (2, 1, 16, 48, 32), (3, 1, 16, 40, 32), (7, 1, 16, 256, 128), (0, 1, 5000, 256, 128),
])
def test_schema_rejects(args):
    with pytest.raises(oes.OesError) as ei:
        oes.schema_make(*args)
    assert ei.value.status == oes.ERR_ARG


def test_null_and_range_errors_without_gpu(L):
    sc = oes.schema_make("bf16", 1, 16, 256, 128)
    out = ctypes.c_void_p()
    assert L.oes_cache_create(None, 8, 0, ctypes.byref(out)) == oes.ERR_ARG
    assert L.oes_cache_create(ctypes.byref(sc), 0, 0, ctypes.byref(out)) == oes.ERR_ARG
    assert L.oes_cache_create(ctypes.byref(sc), 5000, 0, ctypes.byref(out)) == oes.ERR_ARG
    bad = oes.Schema.from_buffer_copy(sc)
    bad.bank[0].row_bytes += 16
    assert L.oes_cache_create(ctypes.byref(bad), 8, 0, ctypes.byref(out)) == oes.ERR_ARG
    assert b"modified" in L.oes_last_error()
    assert L.oes_cache_destroy(None) == oes.OK
    for fn, args in [
        (L.oes_cache_set_source, (None, 0, 0, None, 0)),
        (L.oes_copy_missing, (None, None)),
        (L.oes_ensure_experts, (None, 0, None, 1, 1, None, None)),
        (L.oes_expert_ffn, (None, None, None, None, 1, 1, None, None, 0, None)),
        (L.oes_expert_ffn_noalloc, (None, None, None, None, 1, 1, None, None)),
        (L.oes_cache_check, (None, None)),
        (L.oes_layers_prefetch, (None, 0, None)),
        (L.oes_layers_ffn, (None, 0, None, None, None, 1, 1, None, None, 0, None)),
    ]:
        assert fn(*args) == oes.ERR_ARG
    ws = ctypes.c_int64()
    assert L.oes_route_workspace(4, 2048, 128, ctypes.byref(ws)) == oes.OK and ws.value > 0
    # route argument checks happen before any GPU work
    assert L.oes_route(None, None, 1, 64, 12, 2, None, None, None, None, 0, None) == oes.ERR_ARG  # E not a multiple of 8
    assert L.oes_route(None, None, 1, 64, 16, 0, None, None, None, None, 0, None) == oes.ERR_ARG  # k = 0
    assert L.oes_route(None, None, 1, 64, 16, 17, None, None, None, None, 0, None) == oes.ERR_ARG  # k > E
    assert L.oes_route(None, None, 0, 64, 16, 2, None, None, None, None, 0, None) == oes.OK       # empty
    assert L.oes_route_logits(None, 2, 16, 2, None, None, None) == oes.ERR_ARG
    assert L.oes_debug_decode(oes.ELEM_U8, None, 4, None, None) == oes.ERR_ARG


def test_noalloc_scratch_size_matches_the_header():
    import re
    text = open(oes.HEADER_PATH).read()
    m = re.search(r"#define OES_FFN_NOALLOC_SCRATCH_BYTES \((\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == oes.FFN_NOALLOC_SCRATCH_BYTES


def test_header_lists_binding_functions():
    # every binding entry is declared in the header (no private entry points)
    assert set(oes._SIGS) == set(oes.header_functions())


def test_hybrid_decide_matches_the_oracle_rule():
    """oes_hybrid_decide is host logic: the backend choice and the fetch fraction
    equal the oracle's (benchmark guide §5.2 and §5.4) on a grid of bandwidths."""
    from oracle import formulas
    for fmt in ("bf16", "nvfp4", "q4_0", "fp8_block128", "mxfp4_t"):
        for cpu in (0.0, 20.0, 56.0, 111.9, 112.0, 112.1, 300.0):
            for pcie in (28.0, 56.0):
                for thr in (1.0, 2.0, 3.0):
                    hyb, frac = oes.hybrid_decide(fmt, cpu, pcie, thr)
                    assert hyb == (formulas.recommend_backend(fmt, cpu, pcie, thr) == "hybrid")
                    assert frac == formulas.hybrid_fetch_fraction(pcie, cpu)
    with pytest.raises(oes.OesError):
        oes.hybrid_decide("bf16", 10.0, 0.0)
