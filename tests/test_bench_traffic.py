"""The benchmark's counter-based traffic fields, on the CPU.

Every `traffic <key> bytes_per_launch=.. source=.. sha256=..` line under profiles/
must parse, name an existing source file and use a key no other line uses; the
benchmark reads a value only while that source file still has the recorded hash.
Keys of the decode FFN carry the workload name, so two workloads of one format never
share counters.
"""
import glob
import hashlib
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lines():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            f = line.split()
            if f and f[0] == "traffic":
                out.append((path, f))
    return out


def test_traffic_lines_parse_and_keys_are_unique():
    lines = _lines()
    assert lines, "no traffic lines under profiles/"
    keys = [f[1] for _, f in lines]
    assert len(keys) == len(set(keys)), keys
    for path, f in lines:
        assert len(f) == 5, (path, f)
        kv = dict(x.split("=", 1) for x in f[2:])
        assert set(kv) == {"bytes_per_launch", "source", "sha256"}, (path, f)
        assert int(kv["bytes_per_launch"]) > 0
        assert os.path.exists(os.path.join(ROOT, kv["source"])), kv["source"]
        assert len(kv["sha256"]) == 64


def test_bench_reads_only_current_sources():
    for _, f in _lines():
        kv = dict(x.split("=", 1) for x in f[2:])
        src = os.path.join(ROOT, kv["source"])
        current = hashlib.sha256(open(src, "rb").read()).hexdigest() == kv["sha256"]
        got = bench._pmc_traffic(f[1])
        assert got == (int(kv["bytes_per_launch"]) if current else None), f[1]
    assert bench._pmc_traffic("no_such_kernel") is None


def test_ffn_keys_are_per_workload():
    from synth.workloads import WORKLOADS
    keys = {f[1] for _, f in _lines() if f[1].startswith("expert_ffn_")}
    names = set(WORKLOADS)
    for k in keys:
        rest = k[len("expert_ffn_"):]
        base = rest.rsplit("_bs", 1)[0] if "_bs" in rest else rest
        assert base in names, k
