"""Offloaded expert slots on MI355X: Python binding of liboes.so.

Argument marshalling only: every step of the path runs in the HIP library
(``liboes.so``, built in-tree by ``__graft_entry__.build()`` or
``python offloaded_expert_slot_amd/csrc/build.py``).  PyTorch supplies device
memory and streams; tensors are passed to the C ABI as raw pointers.  If the
library is missing, every call raises - there is no fallback.

The names follow the C ABI in ``include/oes.h``:

    schema_make(format, L, E, H, I)            -> Schema
    Cache(schema, num_slots, device)           .set_source / .set_state / .get_state
                                               .ensure_experts / .copy_missing / .expert_ffn / .resize
    route(x, wg, k, ...) / route_logits(logits, k, ...)
    Layers(schema, depth, device)              .set_source / .prefetch / .ffn
    CpuMoe(schema, threads)                    .set_source / .run   (hybrid backend, host)
    hybrid_decide(format, cpu, pcie) / combine_cpu(y, y_cpu)
"""
import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboes.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "oes.h")

BF16, FP8_BLOCK128, NVFP4, MXFP4_T, Q4_0 = 0, 1, 2, 3, 4
FORMAT_IDS = {"bf16": BF16, "fp8_block128": FP8_BLOCK128, "nvfp4": NVFP4, "mxfp4_t": MXFP4_T, "q4_0": Q4_0}
ELEM_BF16, ELEM_E4M3, ELEM_F32, ELEM_FP4X2, ELEM_FP16, ELEM_E8M0, ELEM_U8, ELEM_Q4X2 = range(8)
OPT_FUSED_COPY, OPT_COPY_MODE, OPT_COPY_BLOCKS, OPT_FFN_PATH = 1, 2, 3, 4
FFN_AUTO, FFN_PER_PAIR, FFN_GROUPED = 0, 1, 2
COPY_ZERO, COPY_SDMA = 0, 1
OK, ERR_ARG, ERR_CAPACITY, ERR_HIP, ERR_NOMEM, ERR_STATE, ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
FFN_NOALLOC_SCRATCH_BYTES = 16 << 20   # OES_FFN_NOALLOC_SCRATCH_BYTES of include/oes.h
MAX_BANKS = 6
MAX_SLOTS = 4096


class OesError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class BankSpec(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("elem", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("row_bytes", ctypes.c_int64)]


class Schema(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_layers", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_banks", ctypes.c_int32),
                ("bank", BankSpec * MAX_BANKS), ("bytes_per_expert", ctypes.c_int64)]

    @property
    def banks(self):
        return [self.bank[i] for i in range(self.num_banks)]

    def bank_names(self):
        return [b.name.decode() for b in self.banks]

    def row_bytes(self):
        return [int(b.row_bytes) for b in self.banks]


class Stats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_uint64), ("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64),
                ("evictions", ctypes.c_uint64), ("bytes_copied", ctypes.c_uint64),
                ("last_misses", ctypes.c_uint32), ("failed_steps", ctypes.c_int32),
                ("last_indices", ctypes.c_uint32), ("last_missing_full", ctypes.c_uint32),
                ("cpu_experts", ctypes.c_uint64)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _U8, _U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint8, ctypes.c_uint64
_PI32, _PI64, _PU64 = ctypes.POINTER(_I32), ctypes.POINTER(_I64), ctypes.POINTER(_U64)
_PF = ctypes.POINTER(ctypes.c_float)

_SIGS = {
    "oes_status_str": (ctypes.c_char_p, [_I32]),
    "oes_last_error": (ctypes.c_char_p, []),
    "oes_abi_version": (_I32, []),
    "oes_schema_make": (_I32, [_I32, _I32, _I32, _I32, _I32, ctypes.POINTER(Schema)]),
    "oes_cache_create": (_I32, [ctypes.POINTER(Schema), _I32, _I32, ctypes.POINTER(_P)]),
    "oes_cache_destroy": (_I32, [_P]),
    "oes_cache_set_source": (_I32, [_P, _I32, _I32, _P, _I64]),
    "oes_cache_set_state": (_I32, [_P, _PI64, _PU64, _U64, _P]),
    "oes_cache_get_state": (_I32, [_P, _PI64, _PU64, _PU64, _P]),
    "oes_cache_snapshot": (_I32, [_P, _P]),
    "oes_cache_restore": (_I32, [_P, _P]),
    "oes_cache_load_rows": (_I32, [_P, _PI32, _PI64, _I32, _P]),
    "oes_cache_fill_slots": (_I32, [_P, _U8, _P]),
    "oes_cache_slot_bank": (_I32, [_P, _I32, ctypes.POINTER(_P), _PI64]),
    "oes_cache_info": (_I32, [_P, _PI32, ctypes.POINTER(Schema)]),
    "oes_cache_get_misses": (_I32, [_P, _PI32, _PI32, _PI64, _I32, _P]),
    "oes_cache_stats": (_I32, [_P, ctypes.POINTER(Stats), _P]),
    "oes_cache_check": (_I32, [_P, _P]),
    "oes_cache_set_option": (_I32, [_P, _I32, _I64]),
    "oes_route_workspace": (_I32, [_I32, _I32, _I32, _PI64]),
    "oes_route": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _I64, _P]),
    "oes_route_logits": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "oes_ensure_experts": (_I32, [_P, _I32, _P, _I32, _I32, _P, _P]),
    "oes_ensure_experts_hybrid": (_I32, [_P, _I32, _P, _I32, _I32, _P, _I32, ctypes.c_double, _P]),
    "oes_copy_missing": (_I32, [_P, _P]),
    "oes_expert_ffn_workspace": (_I32, [_P, _I32, _I32, _PI64]),
    "oes_expert_ffn": (_I32, [_P, _P, _P, _P, _I32, _I32, _P, _P, _I64, _P]),
    "oes_expert_ffn_noalloc": (_I32, [_P, _P, _P, _P, _I32, _I32, _P, _P]),
    "oes_layers_create": (_I32, [ctypes.POINTER(Schema), _I32, _I32, ctypes.POINTER(_P)]),
    "oes_layers_destroy": (_I32, [_P]),
    "oes_layers_set_source": (_I32, [_P, _I32, _I32, _P, _I64]),
    "oes_layers_prefetch": (_I32, [_P, _I32, _P]),
    "oes_layers_buffer": (_I32, [_P, _I32, _I32, ctypes.POINTER(_P), _PI64]),
    "oes_layers_ffn_workspace": (_I32, [_P, _I32, _I32, _PI64]),
    "oes_layers_ffn": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _P, _P, _I64, _P]),
    "oes_probe_h2d_dma": (_I32, [_P, _P, _I64, _P, _PF]),
    "oes_probe_h2d_kernel": (_I32, [_P, _P, _I64, _I32, _P, _PF]),
    "oes_probe_hbm_read": (_I32, [_P, _I64, _I64, _I32, _P, _P, _PF]),
    "oes_probe_mfma_bf16": (_I32, [_I32, _I32, _P, _P, _PF, ctypes.POINTER(ctypes.c_double)]),
    "oes_probe_mfma_f8f4": (_I32, [_I32, _I32, _P, _P, _PF, ctypes.POINTER(ctypes.c_double)]),
    "oes_debug_decode": (_I32, [_I32, _P, _I32, _P, _P]),
    "oes_cache_resize": (_I32, [_P, _I32, _P]),
    "oes_cpu_moe_create": (_I32, [ctypes.POINTER(Schema), _I32, ctypes.POINTER(_P)]),
    "oes_cpu_moe_destroy": (_I32, [_P]),
    "oes_cpu_moe_threads": (_I32, [_P, _PI32]),
    "oes_cpu_moe_set_source": (_I32, [_P, _I32, _I32, _P, _I64]),
    "oes_cpu_moe_run": (_I32, [_P, _I32, _P, _P, _P, _P, _I32, _I32, _P]),
    "oes_cpu_moe_probe_read": (_I32, [_P, _P, _I64, ctypes.POINTER(ctypes.c_double)]),
    "oes_hybrid_decide": (_I32, [_I32, ctypes.c_double, ctypes.c_double, ctypes.c_double, _PI32,
                                 ctypes.POINTER(ctypes.c_double)]),
    "oes_combine_cpu": (_I32, [_P, _P, _I64, _P]),
    "oes_hybrid_workspace": (_I32, [_P, _I32, _I32, _PI64, _PI64]),
    "oes_hybrid_step": (_I32, [_P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P, _I64, _P, _I64, _I32,
                               ctypes.c_double, _P]),
}


def lib():
    """Load liboes.so once; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OesError(ERR_STATE, f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/oes.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oes_[a-z0-9_]+)\s*\(", text)))


def _check(status):
    if status != OK:
        L = lib()
        raise OesError(status, f"{L.oes_status_str(status).decode()}: {L.oes_last_error().decode()}")


def _ptr(t):
    """Raw address of a tensor / array / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    raise TypeError(type(t))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def schema_make(fmt, num_layers, num_experts, hidden, inter):
    if isinstance(fmt, str):
        fmt = FORMAT_IDS[fmt]
    sc = Schema()
    _check(lib().oes_schema_make(fmt, num_layers, num_experts, hidden, inter, ctypes.byref(sc)))
    return sc


def _device_view(addr, nbytes, device):
    """torch uint8 tensor over library-owned device memory (no copy)."""
    import torch

    class _View:
        __cuda_array_interface__ = {"shape": (int(nbytes),), "typestr": "|u1", "data": (int(addr), False),
                                    "version": 2}
    return torch.as_tensor(_View(), device=f"cuda:{device}")


class Cache:
    """Slot cache: HBM slot banks + LRU table (oes_cache_*)."""

    def __init__(self, schema, num_slots, device=0):
        self.schema = schema
        self.num_slots = num_slots
        self.device = device
        h = _P()
        _check(lib().oes_cache_create(ctypes.byref(schema), num_slots, device, ctypes.byref(h)))
        self._h = h
        self._sources = {}

    def close(self):
        if self._h:
            _check(lib().oes_cache_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def set_source(self, bank, layer, host_tensor):
        _check(lib().oes_cache_set_source(self._h, bank, layer, _ptr(host_tensor), host_tensor.numel() *
                                          host_tensor.element_size()))
        self._sources[(bank, layer)] = host_tensor  # keep alive

    def set_option(self, option, value):
        _check(lib().oes_cache_set_option(self._h, option, int(value)))

    def set_state(self, owner, stamp, clock=0, stream=None):
        owner = np.ascontiguousarray(owner, dtype=np.int64)
        stamp = np.ascontiguousarray(stamp, dtype=np.uint64)
        _check(lib().oes_cache_set_state(self._h, owner.ctypes.data_as(_PI64), stamp.ctypes.data_as(_PU64),
                                         int(clock), _stream(stream)))

    def get_state(self, stream=None):
        owner = np.empty(self.num_slots, dtype=np.int64)
        stamp = np.empty(self.num_slots, dtype=np.uint64)
        clock = _U64()
        _check(lib().oes_cache_get_state(self._h, owner.ctypes.data_as(_PI64), stamp.ctypes.data_as(_PU64),
                                         ctypes.byref(clock), _stream(stream)))
        return owner, stamp, int(clock.value)

    def resize(self, num_slots, stream=None):
        """Grow or shrink the slot pool in place (resident experts and their LRU order kept)."""
        _check(lib().oes_cache_resize(self._h, int(num_slots), _stream(stream)))
        self.num_slots = int(num_slots)

    def snapshot(self, stream=None):
        _check(lib().oes_cache_snapshot(self._h, _stream(stream)))

    def restore(self, stream=None):
        _check(lib().oes_cache_restore(self._h, _stream(stream)))

    def load_rows(self, slots, ids, stream=None):
        slots = np.ascontiguousarray(slots, dtype=np.int32)
        ids = np.ascontiguousarray(ids, dtype=np.int64)
        _check(lib().oes_cache_load_rows(self._h, slots.ctypes.data_as(_PI32), ids.ctypes.data_as(_PI64),
                                         len(slots), _stream(stream)))

    def fill_slots(self, value, stream=None):
        _check(lib().oes_cache_fill_slots(self._h, value, _stream(stream)))

    def slot_bank(self, bank):
        """(device address, row bytes) of slot bank `bank`."""
        base, rb = _P(), _I64()
        _check(lib().oes_cache_slot_bank(self._h, bank, ctypes.byref(base), ctypes.byref(rb)))
        return base.value, rb.value

    def slot_bank_view(self, bank):
        """uint8 [S, row_bytes] torch view of slot bank `bank` (library-owned memory)."""
        base, rb = self.slot_bank(bank)
        return _device_view(base, self.num_slots * rb, self.device).view(self.num_slots, rb)

    def get_misses(self, stream=None):
        cap = self.num_slots
        n = _I32()
        slots = np.empty(cap, dtype=np.int32)
        ids = np.empty(cap, dtype=np.int64)
        _check(lib().oes_cache_get_misses(self._h, ctypes.byref(n), slots.ctypes.data_as(_PI32),
                                          ids.ctypes.data_as(_PI64), cap, _stream(stream)))
        return list(zip(slots[:n.value].tolist(), ids[:n.value].tolist()))

    def stats(self, stream=None):
        st = Stats()
        _check(lib().oes_cache_stats(self._h, ctypes.byref(st), _stream(stream)))
        return {f: getattr(st, f) for f, _ in Stats._fields_}

    def check(self, stream=None):
        """Raises OesError for a sticky device error (capacity / bad id)."""
        _check(lib().oes_cache_check(self._h, _stream(stream)))

    def check_status(self, stream=None):
        return lib().oes_cache_check(self._h, _stream(stream))

    # ---- the step
    def ensure_experts(self, layer, ids, slot_ids, stream=None):
        n, k = ids.shape
        _check(lib().oes_ensure_experts(self._h, layer, _ptr(ids), n, k, _ptr(slot_ids), _stream(stream)))

    def ensure_experts_hybrid(self, layer, ids, slot_ids, max_fetch=-1, fetch_fraction=-1.0, stream=None):
        """Hybrid remap: at most the cap of misses get slots; the rest map to -1."""
        n, k = ids.shape
        _check(lib().oes_ensure_experts_hybrid(self._h, layer, _ptr(ids), n, k, _ptr(slot_ids), int(max_fetch),
                                               float(fetch_fraction), _stream(stream)))

    def hybrid_workspace(self, n, k):
        """(pinned host bytes, device bytes) a hybrid step of n tokens needs."""
        hb, db = _I64(), _I64()
        _check(lib().oes_hybrid_workspace(self._h, n, k, ctypes.byref(hb), ctypes.byref(db)))
        return hb.value, db.value

    def hybrid_step(self, cpu, layer, x, ids, w, slot_ids, y, ffn_ws, host_ws, dev_ws, max_fetch=-1,
                    fetch_fraction=-1.0, stream=None):
        """ensure_experts_hybrid + copy + GPU FFN, the -1 experts on the CPU executor, combined into y."""
        n, k = ids.shape
        _check(lib().oes_hybrid_step(self._h, cpu._h, layer, _ptr(x), _ptr(ids), _ptr(w), n, k, _ptr(slot_ids),
                                     _ptr(y), _ptr(ffn_ws), ffn_ws.numel(), _ptr(host_ws), host_ws.numel(),
                                     _ptr(dev_ws), dev_ws.numel(), int(max_fetch), float(fetch_fraction),
                                     _stream(stream)))

    def copy_missing(self, stream=None):
        _check(lib().oes_copy_missing(self._h, _stream(stream)))

    def ffn_workspace_bytes(self, n, k):
        b = _I64()
        _check(lib().oes_expert_ffn_workspace(self._h, n, k, ctypes.byref(b)))
        return b.value

    def expert_ffn(self, x, slot_ids, w, y, workspace, stream=None):
        n, k = slot_ids.shape
        _check(lib().oes_expert_ffn(self._h, _ptr(x), _ptr(slot_ids), _ptr(w), n, k, _ptr(y), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))

    def expert_ffn_noalloc(self, x, slot_ids, w, y, stream=None):
        """expert_ffn on the library's own per-GPU scratch array (no workspace, no allocation)."""
        n, k = slot_ids.shape
        _check(lib().oes_expert_ffn_noalloc(self._h, _ptr(x), _ptr(slot_ids), _ptr(w), n, k, _ptr(y),
                                            _stream(stream)))


def route_workspace_bytes(n, hidden, num_experts):
    b = _I64()
    _check(lib().oes_route_workspace(n, hidden, num_experts, ctypes.byref(b)))
    return b.value


def route(x, wg, k, ids, w, workspace, logits=None, stream=None):
    n, H = x.shape
    E = wg.shape[1]
    _check(lib().oes_route(_ptr(x), _ptr(wg), n, H, E, k, _ptr(ids), _ptr(w), _ptr(logits), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))


def route_logits(logits, k, ids, w, stream=None):
    n, E = logits.shape
    _check(lib().oes_route_logits(_ptr(logits), n, E, k, _ptr(ids), _ptr(w), _stream(stream)))


class Layers:
    """Whole-layer double buffer for prefill (oes_layers_*)."""

    def __init__(self, schema, depth=2, device=0):
        self.schema = schema
        self.depth = depth
        self.device = device
        h = _P()
        _check(lib().oes_layers_create(ctypes.byref(schema), depth, device, ctypes.byref(h)))
        self._h = h
        self._sources = {}

    def close(self):
        if self._h:
            _check(lib().oes_layers_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_source(self, bank, layer, host_tensor):
        _check(lib().oes_layers_set_source(self._h, bank, layer, _ptr(host_tensor),
                                           host_tensor.numel() * host_tensor.element_size()))
        self._sources[(bank, layer)] = host_tensor

    def prefetch(self, layer, copy_stream=None):
        _check(lib().oes_layers_prefetch(self._h, layer, _stream(copy_stream)))

    def buffer_view(self, index, bank):
        dev, nbytes = _P(), _I64()
        _check(lib().oes_layers_buffer(self._h, index, bank, ctypes.byref(dev), ctypes.byref(nbytes)))
        return _device_view(dev.value, nbytes.value, self.device)

    def ffn_workspace_bytes(self, n, k):
        b = _I64()
        _check(lib().oes_layers_ffn_workspace(self._h, n, k, ctypes.byref(b)))
        return b.value

    def ffn(self, layer, x, ids, w, y, workspace, stream=None):
        n, k = ids.shape
        _check(lib().oes_layers_ffn(self._h, layer, _ptr(x), _ptr(ids), _ptr(w), n, k, _ptr(y), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


class CpuMoe:
    """CPU MoE executor of the hybrid backend (oes_cpu_moe_*): host tensors only."""

    def __init__(self, schema, threads=0):
        self.schema = schema
        h = _P()
        _check(lib().oes_cpu_moe_create(ctypes.byref(schema), int(threads), ctypes.byref(h)))
        self._h = h
        self._sources = {}

    def close(self):
        if self._h:
            _check(lib().oes_cpu_moe_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def threads(self):
        n = _I32()
        _check(lib().oes_cpu_moe_threads(self._h, ctypes.byref(n)))
        return n.value

    def set_source(self, bank, layer, host_tensor):
        _check(lib().oes_cpu_moe_set_source(self._h, bank, layer, _ptr(host_tensor),
                                            host_tensor.numel() * host_tensor.element_size()))
        self._sources[(bank, layer)] = host_tensor  # keep alive

    def run(self, layer, x, ids, slot_ids, w, y):
        """y[n, H] fp32 = the experts of the pairs with slot_ids < 0 (host tensors or arrays)."""
        n, k = ids.shape
        _check(lib().oes_cpu_moe_run(self._h, layer, _ptr(x), _ptr(ids), _ptr(slot_ids), _ptr(w), n, k, _ptr(y)))

    def probe_read(self, buf, nbytes):
        """Wall ms of reading nbytes of a host buffer with every thread."""
        ms = ctypes.c_double()
        _check(lib().oes_cpu_moe_probe_read(self._h, _ptr(buf), int(nbytes), ctypes.byref(ms)))
        return ms.value


def hybrid_decide(fmt, cpu_gbps, pcie_gbps, threshold=2.0):
    """(use hybrid?, fetch fraction) of the measured bandwidths (oes_hybrid_decide)."""
    h, f = _I32(), ctypes.c_double()
    _check(lib().oes_hybrid_decide(FORMAT_IDS.get(fmt, fmt), float(cpu_gbps), float(pcie_gbps), float(threshold),
                                   ctypes.byref(h), ctypes.byref(f)))
    return bool(h.value), f.value


def combine_cpu(y, y_cpu, stream=None):
    """y (bf16 bits, device) += y_cpu (fp32, device), rounded to bf16."""
    _check(lib().oes_combine_cpu(_ptr(y), _ptr(y_cpu), y.numel(), _stream(stream)))


def debug_decode(elem, codes, n, out, stream=None):
    _check(lib().oes_debug_decode(elem, _ptr(codes), n, _ptr(out), _stream(stream)))


def probe_h2d_dma(dev, host, nbytes, stream=None):
    ms = ctypes.c_float()
    _check(lib().oes_probe_h2d_dma(_ptr(dev), _ptr(host), nbytes, _stream(stream), ctypes.byref(ms)))
    return ms.value


def probe_h2d_kernel(dev, host, nbytes, blocks=1024, stream=None):
    ms = ctypes.c_float()
    _check(lib().oes_probe_h2d_kernel(_ptr(dev), _ptr(host), nbytes, blocks, _stream(stream), ctypes.byref(ms)))
    return ms.value


def probe_hbm_read(dev, nbytes, sink, stride=0, count=1, stream=None):
    """ms per read of `count` back-to-back streaming reads of nbytes, the i-th at dev + i*stride."""
    ms = ctypes.c_float()
    _check(lib().oes_probe_hbm_read(_ptr(dev), nbytes, stride, count, _ptr(sink), _stream(stream), ctypes.byref(ms)))
    return ms.value


def probe_mfma_bf16(blocks, iters, sink, stream=None):
    """(ms, flops) of the bf16 MFMA loop: blocks x 4 waves x iters x 4 chained 32x32x16 MFMAs."""
    ms, flops = ctypes.c_float(), ctypes.c_double()
    _check(lib().oes_probe_mfma_bf16(blocks, iters, _ptr(sink), _stream(stream), ctypes.byref(ms), ctypes.byref(flops)))
    return ms.value, flops.value


def probe_mfma_f8f4(blocks, iters, sink, stream=None):
    """(ms, flops) of the block-scaled e4m3 x e2m1 MFMA loop (32x32x64), the prefill GEMM's instruction."""
    ms, flops = ctypes.c_float(), ctypes.c_double()
    _check(lib().oes_probe_mfma_f8f4(blocks, iters, _ptr(sink), _stream(stream), ctypes.byref(ms), ctypes.byref(flops)))
    return ms.value, flops.value
