"""The CPU MoE executor (host C++, hybrid backend) built on its own with the
address and undefined-behaviour sanitizers and run on this host's CPU against
the oracle: the same sources as liboes.so (cpu_moe.cpp, host_common.cpp) plus
a test driver (tests/sanitize/cpu_moe_driver.cpp) that runs one step at several
thread counts and walks the argument errors.  Any sanitizer report ends the
driver with a non-zero status.

Needs g++ and a CPU with AVX-512 F/BW/VL/BF16 (the executor's instructions);
skipped otherwise.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest
import torch

import synth
from oracle import ffn as offn
from synth.workloads import Workload, make_host_banks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "offloaded_expert_slot_amd", "csrc")
FORMATS = {"bf16": 0, "nvfp4": 2, "q4_0": 4}


def _cpu_ok():
    if shutil.which("g++") is None:
        return False
    try:
        flags = open("/proc/cpuinfo").read()
    except OSError:
        return False
    return all(f in flags for f in ("avx512f", "avx512bw", "avx512vl", "avx512_bf16", "f16c"))


pytestmark = pytest.mark.skipif(not _cpu_ok(), reason="needs g++ and AVX-512 BF16 on the host")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asan") / "cpu_moe_asan")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "cpu_moe.cpp"), os.path.join(CSRC, "host_common.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "cpu_moe_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _write_case(path, fmt, E, H, I, x, ids, slots, w, threads, banks):
    n, k = ids.shape
    with open(path, "wb") as f:
        f.write(struct.pack("<7i", FORMATS[fmt], E, H, I, n, k, len(threads)))
        f.write(struct.pack(f"<{len(threads)}i", *threads))
        f.write(struct.pack("<i", len(banks)))
        for b in banks:
            raw = b.numpy().tobytes()
            f.write(struct.pack("<q", len(raw)))
            f.write(raw)
        f.write(x.numpy().view(np.uint16).tobytes())
        f.write(ids.astype(np.int32).tobytes())
        f.write(slots.astype(np.int32).tobytes())
        f.write(w.astype(np.float32).tobytes())


@pytest.mark.parametrize("fmt,H,I,E,n,k", [
    ("bf16", 256, 128, 6, 3, 4),
    ("bf16", 264, 136, 5, 2, 3),     # K not a multiple of 32: the masked tail
    ("nvfp4", 512, 256, 6, 2, 3),    # even/odd operand split
    ("nvfp4", 288, 160, 5, 2, 3),    # element-order path
    ("q4_0", 512, 256, 6, 3, 4),
])
def test_cpu_moe_sanitized(driver, tmp_path, fmt, H, I, E, n, k):
    hb = make_host_banks(Workload(f"asan-{fmt}-{H}", fmt, L=1, E=E, k=1, H=H, I=I, S=1), device="cpu", pin=False)
    rng = np.random.default_rng(H + n)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    slots = np.where(rng.random((n, k)) < 0.6, -1, 3).astype(np.int32)
    slots[0, 0] = -1
    slots[n - 1] = 2                  # a token with no CPU pair: its y row is 0
    w = rng.random((n, k)).astype(np.float32)
    x = synth.activations(n, H, 0, f"asan-{fmt}")
    threads = [1, 3, 4]
    inp, out = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    _write_case(inp, fmt, E, H, I, x, ids, slots, w, threads, hb.banks)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver, inp, out], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    ys = np.fromfile(out, dtype=np.float32).reshape(len(threads), n, H)
    # the summation order does not depend on the thread count
    assert all(np.array_equal(ys[0], ys[i]) for i in range(1, len(threads)))
    rows = lambda e: [hb.row(b, int(e)).numpy() for b in range(len(hb.banks))]
    ref = offn.expert_ffn(fmt, H, I, x.numpy().view(np.uint16), np.where(slots < 0, ids, -1), w.astype(np.float64),
                          rows)
    err = offn.rel_l2(ys[0].astype(np.float64), ref)
    assert err <= 5e-3, err
    assert (ys[0][n - 1] == 0).all()
