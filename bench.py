"""Benchmark of the per-layer offloaded-expert MoE step on one MI355X.

Metric: copy_missing GB/s + tok_ms per miss rate; MoE-layer decode tok/s at bs=1.

Headline workload: bf16 banks, H=2048, I=768, E=128 experts, top-8, L=48 MoE
layers, a 1024-slot pool whose every slot starts owned by another layer;
layer 0 is driven and per-token costs are extrapolated over L layers (FreeToken
MoE benchmark guide §4.3-§4.4).  Inputs are seeded synthetic tensors resident
in HBM (activations, router) and in pinned host banks (experts).

One "step" = route -> ensure_experts -> copy_missing -> expert_ffn for one
token (bs=1), with the slot table restored on the device (untimed) before each
step so that misses = round(active * miss_rate) of the routed experts miss.
Steps are enqueued back to back and each is timed with HIP events on the
launch stream at its two ends; value = 1000 / (L * ms_per_step) at the
headline miss rate.  A second pass with events between the four parts gives
the breakdown and the copy's time.

Every workload is measured the same way (`configs` in the JSON line): the tiny
bf16 one (H=256, 16 experts, top-2, 8 slots, bs 1 and 4), bf16 H=2048, block
fp8 H=4096 (256 experts, 2048 slots), NVFP4 H=7168 (256 experts, 1536 slots),
GGUF Q4_0 at the bf16 model's shape, and the MXFP4 prefill layer:
  * the copy sweep in the benchmark guide's columns (bs, active, miss_rate,
    misses, time_ms, copy_MiB, bw_GBps, tok_ms), the median of 25 event-timed
    ensure+copy repeats for the fused gather, one launch per bank, and the DMA
    mode (which reads the miss list on the host);
  * the decode step at every miss rate of the workload;
  * the expert FFN alone, cold (each launch on experts no earlier launch of
    the loop read), at bs=1 and at the workload's larger batches, against the
    HBM roofline of the unique experts' bytes;
  * each row's step checked against the CPU oracle on the same inputs (routed
    ids, slot map, miss list, the missed rows' bytes in every bank, the FFN
    output within the format's tolerance), with the oracle's own route, LRU,
    copy and FFN times on this host.
Also: the measured ceilings (pinned H2D by DMA and by the zero-copy kernel,
HBM streaming read, the bf16 and the block-scaled e4m3 x e2m1 MFMA loops), the
hybrid backend (host DRAM read and link ceilings, the CPU MoE executor and the
PCIe gather alone and overlapped, the decision and fetch split, the hybrid
decode layer step beside the offload one), a slot-pool resize, the MXFP4
prefill layer (grouped FFN on the block-scaled MFMA, whole-layer stream, the
overlapped loop over 4 layers) and the oracle's headline step timed as the CPU
baseline.  A row that differs from the oracle makes the run invalid: the line
says so and the exit status is 1.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "copy_missing GB/s + tok_ms per miss rate; MoE-layer decode tok/s at bs=1"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
PCIE_PEAK_GBS = 64.0         # PCIe 5.0 x16, one direction, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
DECODE_CONFIGS = ("bf16_tiny", "bf16_h2048", "fp8_h4096", "nvfp4_h7168", "q4_0_h2048")
FP4_FORMATS = ("nvfp4", "q4_0", "mxfp4_t")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bf16_h2048", help="headline workload")
    ap.add_argument("--miss-rate", type=float, default=0.5, help="headline miss rate")
    ap.add_argument("--repeat", type=int, default=25, help="repeats per copy-sweep row (median)")
    ap.add_argument("--configs", default=",".join(DECODE_CONFIGS + ("mxfp4_prefill",)),
                    help="comma-separated workloads measured besides the headline one")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-sdma", action="store_true", help="skip the DMA-mode column of the copy sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-hybrid", action="store_true", help="skip the hybrid backend (CPU executor) part")
    ap.add_argument("--hybrid-steps", type=int, default=20, help="timed hybrid / synced offload layer steps")
    return ap.parse_args()


def _r(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the step has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth.workloads import WORKLOADS

    torch.cuda.set_device(torch.device("cuda:0"))
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731
    head_w = WORKLOADS[args.workload]
    probes = {} if args.no_probes else _probes(head_w, log)

    # ---------------------------------------------------------------- headline workload
    head, ctx = _decode_config(args.workload, args, probes, log, headline=True)
    hrow = ctx["headline_row"]
    hybrid = None
    if not args.no_hybrid:
        hybrid = _hybrid(ctx["cache"], ctx["hb"], head_w, ctx["bpe"], ctx["x"], ctx["wg"], ctx["rws"], ctx["fws"],
                         ctx["prepare"], probes, head["decode"], args, log)
    resize = _resize(ctx["cache"], head_w, ctx["bpe"], log)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(head_w, ctx["hb"], ctx["x"], ctx["wg"], args.miss_rate, args.cpu_seconds)
        log("cpu_baseline", cpu)
    ctx["cache"].close()
    del ctx
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- the other workloads
    configs = {args.workload: head}
    prefill = None
    for name in [c for c in args.configs.split(",") if c and c != args.workload]:
        if name == "mxfp4_prefill":
            prefill = _prefill(WORKLOADS[name], probes, log)
            configs[name] = prefill
        else:
            configs[name], c2 = _decode_config(name, args, probes, log, headline=False)
            c2["cache"].close()
            del c2
            torch.cuda.empty_cache()
    if hybrid is not None:
        pcie = {n: _best_copy_GBps(c) for n, c in configs.items() if n != "mxfp4_prefill"}
        hybrid["formats"] = _cpu_formats(WORKLOADS, pcie, log)

    # ---------------------------------------------------------------- rooflines
    kernels = {}
    ffn1 = head["ffn"]["bs1"]
    kernels["expert_ffn"] = {"bound": "hbm", "achieved": ffn1["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": ffn1["GBps"] / HBM_PEAK_GBS, "bytes_per_launch": ffn1["bytes"],
                             "avg_ms": ffn1["avg_ms"], "traffic": ffn1["traffic"]}
    if probes:
        kernels["expert_ffn"]["frac_of_measured_hbm_read"] = ffn1["GBps"] / probes["hbm_read_GBps"]
    if hrow["misses"]:
        cbytes = hrow["misses"] * ctx_bpe(head)
        cgbs = cbytes / (hrow["copy_ms"] * 1e6)
        kernels["copy_missing"] = {"bound": "host_link", "achieved": cgbs, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                                   "frac": cgbs / PCIE_PEAK_GBS, "bytes_per_launch": cbytes,
                                   "avg_ms": hrow["copy_ms"], "traffic": _pmc_traffic("copy_missing")}
        if probes:
            kernels["copy_missing"]["frac_of_measured_h2d_peak"] = cgbs / probes["h2d_peak_GBps"]
    dominant = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    rk = kernels[dominant]
    roof = {"kernel": dominant, "bound": rk["bound"], "achieved": rk["achieved"], "peak": rk["peak"],
            "unit": rk["unit"], "frac": rk["frac"], "traffic": rk["traffic"]}
    if prefill is not None:
        kernels["prefill_ffn"] = {"bound": "mfma", "achieved": prefill["ffn_TFLOPs"], "peak": BF16_MFMA_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": prefill["ffn_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS,
                                  "flops_per_launch": prefill["flops"], "avg_ms": prefill["ffn_ms"],
                                  "hbm_GBps": prefill["ffn_weight_GBps"], "traffic": _pmc_traffic("prefill_ffn")}
        # the min(MFMA, HBM x intensity) roofline: 407.7 GFLOP over 1.694 GB of weights
        ridge = min(BF16_MFMA_PEAK_TFLOPS, HBM_PEAK_GBS * prefill["flops"] / prefill["layer_bytes"] / 1e3)
        kernels["prefill_ffn"]["min_roofline_TFLOPs"] = ridge
        kernels["prefill_ffn"]["frac_of_min_roofline"] = prefill["ffn_TFLOPs"] / ridge
        kernels["prefill_ffn"]["instruction"] = prefill["instruction"]
        if probes:
            ceiling = probes["mfma_f8f4_TFLOPs"] / 2.0
            kernels["prefill_ffn"]["measured_mfma_ceiling_TFLOPs"] = ceiling
            kernels["prefill_ffn"]["frac_of_measured_mfma_peak"] = prefill["ffn_TFLOPs"] / ceiling

    # ---------------------------------------------------------------- parity over every row
    failed = [(n, r.get("what", "row")) for n, c in configs.items() for r in _rows_of(c)
              if r.get("parity") is not None and not r["parity"]["ok"]]
    parity = {"ok": not failed, "rows_checked": sum(1 for c in configs.values() for r in _rows_of(c)
                                                    if r.get("parity") is not None),
              "failed": failed, "headline": hrow["parity"],
              "configs": {n: all(r["parity"]["ok"] for r in _rows_of(c) if r.get("parity") is not None)
                          for n, c in configs.items()}}
    ms = hrow["ms_per_step"]
    out = {
        "metric": METRIC, "value": 1000.0 / (head_w.L * ms), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head_w.name, "format": head_w.fmt, "hidden": head_w.H, "inter": head_w.I,
                   "experts": head_w.E, "topk": head_w.k, "layers": head_w.L, "slots": head_w.S, "bs": 1,
                   "miss_rate": args.miss_rate, "misses": hrow["misses"], "active": hrow["active"],
                   "bytes_per_expert": ctx_bpe(head)},
        "tok_ms": hrow["tok_ms"], "copy_GBps": hrow.get("copy_GBps"),
        "roofline": roof, "cpu_baseline": cpu, "parity": parity, "kernels": kernels, "probes": probes,
        "decode_per_miss_rate": head["decode"], "copy_sweep": head["copy_sweep"], "configs": configs,
        "hybrid": hybrid, "resize": resize, "prefill": prefill,
    }
    if not hrow["parity"]["ok"]:
        # a number from a step that does not match the oracle is not reported
        out["value"] = None
    if failed:
        out["invalid"] = f"{len(failed)} measured row(s) differ from the oracle (see parity.failed)"
    print(json.dumps(out), flush=True)
    if failed:
        sys.exit(1)


def ctx_bpe(cfg):
    return cfg["bytes_per_expert"]


def _rows_of(cfg):
    rows = list(cfg.get("decode", [])) + list(cfg.get("copy_sweep", []))
    for key in ("bs1",) + tuple(k for k in cfg.get("ffn", {}) if k.startswith("bs") and k != "bs1"):
        if key in cfg.get("ffn", {}):
            rows.append(cfg["ffn"][key])
    if "gate" in cfg:
        rows.append(cfg["gate"])
    return rows


def _best_copy_GBps(cfg):
    """The fused gather's rate on the sweep row with the most misses."""
    rows = [r for r in cfg.get("copy_sweep", []) if r.get("bw_GBps")]
    return max(rows, key=lambda r: r["misses"])["bw_GBps"] if rows else None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _host_info():
    return {"cpu_model": _cpu_model(), "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "blas_threads": int(_blas_threads()),
            "threads_note": "route, LRU and row copies single-threaded; FFN matmuls on the BLAS threads"}


# ============================================================================ ceilings
def _probes(w, log):
    import torch

    import offloaded_expert_slot_amd as oes

    dev = torch.device("cuda:0")
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    src.fill_(3)
    nbytes = src.numel()
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dma = [oes.probe_h2d_dma(dbuf, src, nbytes) for _ in range(5)]
    zc = [oes.probe_h2d_kernel(dbuf, src, nbytes, 1024) for _ in range(5)]
    big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    big.fill_(1)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    hbm = [oes.probe_hbm_read(big, big.numel(), sink) for _ in range(5)]
    mfma = [oes.probe_mfma_bf16(2048, 10000, sink) for _ in range(3)]
    mfma_f8f4 = [oes.probe_mfma_f8f4(2048, 5000, sink) for _ in range(3)]
    # streaming reads of the bs=1 FFN's byte count of the headline workload, back to
    # back over 16 distinct regions, timed like the FFN alone
    sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
    fb = (w.k * sc.bytes_per_expert // 16) * 16
    fstride = (fb + 4095) // 4096 * 4096
    hbm_small = [oes.probe_hbm_read(big, fb, sink, stride=fstride, count=16) for _ in range(4)]
    probes = {
        "h2d_dma_GBps": nbytes / (min(dma) * 1e6),
        "h2d_zero_copy_GBps": nbytes / (min(zc) * 1e6),
        "hbm_read_GBps": big.numel() / (min(hbm) * 1e6),
        "mfma_bf16_TFLOPs": max(fl / (ms * 1e9) for ms, fl in mfma),
        "mfma_f8f4_TFLOPs": max(fl / (ms * 1e9) for ms, fl in mfma_f8f4),
        "hbm_read_ffn_bytes_GBps": fb / (min(hbm_small) * 1e6),
        "ffn_bytes": fb,
        "h2d_bytes": nbytes,
    }
    probes["h2d_peak_GBps"] = max(probes["h2d_dma_GBps"], probes["h2d_zero_copy_GBps"])
    del big, dbuf, src
    torch.cuda.empty_cache()
    log("probes", _r(probes))
    return probes


# ============================================================================ the oracle side
def _oracle_step(w, host, state, row_bytes, ids=None, xb=None, wgb=None, ffn=True):
    """One step of the oracle from a slot-table state, timed part by part (ms).

    host[b][0] is layer 0's bank b as numpy [E, row_bytes]; state is (owner,
    stamp, clock).  Routed when ids is None (x and Wg given); the FFN reads each
    slot's expert from the host banks through the slot's owner."""
    import numpy as np

    from oracle import copy as ocopy
    from oracle import ffn as offn
    from oracle import route as oroute
    from oracle.lru import SlotTable

    t = {}
    c0 = time.perf_counter()
    wts = None
    if ids is None:
        ids, wts, _ = oroute.route(xb, wgb, w.k)
        t["t_route_ms"] = (time.perf_counter() - c0) * 1e3
    c1 = time.perf_counter()
    table = SlotTable(w.S, w.L, w.E)
    table.set_state(*state)
    r = table.ensure(0, ids)
    c2 = time.perf_counter()
    mirror = [np.zeros((w.S, rb), dtype=np.uint8) for rb in row_bytes]   # pages committed as rows land
    ocopy.copy_missing(r.misses, host, mirror, w.E)
    c3 = time.perf_counter()
    t["t_ensure_ms"] = (c2 - c1) * 1e3
    t["t_copy_ms"] = (c3 - c2) * 1e3
    y = None
    if ffn:
        y = offn.expert_ffn(w.fmt, w.H, w.I, xb, r.slot_ids, wts,
                            lambda s: [host[b][0][int(table.owner[s]) % w.E] for b in range(len(host))])
        t["t_ffn_ms"] = (time.perf_counter() - c3) * 1e3
    t["ms_per_step"] = sum(v for k, v in t.items() if k.startswith("t_"))
    sl = [s for s, _ in r.misses]
    rows = [m[sl].copy() for m in mirror]
    del mirror
    return {"ids": ids, "slot_ids": r.slot_ids, "misses": [(int(s), int(f)) for s, f in r.misses],
            "rows": rows, "y": y, "status": r.status}, t


def _gate(gpu, orc, tol=None, routed=True):
    """Compare one GPU step with the oracle's: routed ids, slot map, miss list
    (install order), the missed rows' bytes of every bank, and the FFN output."""
    import numpy as np

    from oracle import ffn as offn

    res = {}
    if routed:
        res["ids"] = bool(np.array_equal(gpu["ids"], orc["ids"]))
    res["slot_ids"] = bool(np.array_equal(gpu["slot_ids"], orc["slot_ids"]))
    res["misses"] = gpu["misses"] == orc["misses"]
    res["slot_bytes"] = res["misses"] and all(np.array_equal(g, o) for g, o in zip(gpu["rows"], orc["rows"]))
    ok = all(res.values())
    if orc.get("y") is not None:
        err = float(offn.rel_l2(gpu["y"], orc["y"]))
        res["ffn_rel_l2"] = err
        res["ffn_tol"] = tol
        ok = ok and err <= tol
    res["ok"] = bool(ok)
    return res


def _tol(fmt):
    return 3e-2 if fmt in FP4_FORMATS else 1e-2


# ============================================================================ one decode workload
def _decode_config(name, args, probes, log, headline):
    """Copy sweep, decode step per miss rate and the FFN alone of one decode
    workload, every row gated by the oracle.  Returns (results, context); the
    context holds the cache (the caller closes it) and, for the headline
    workload, what the hybrid and resize parts reuse."""
    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth
    from oracle import ffn as offn
    from oracle import formulas
    from synth.workloads import WORKLOADS, make_host_banks

    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    tol = _tol(w.fmt)
    t0 = time.time()
    hb = make_host_banks(w)
    gen_s = time.time() - t0
    sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
    bpe = sc.bytes_per_expert
    cache = oes.Cache(sc, w.S, 0)
    for b, t in enumerate(hb.banks):
        cache.set_source(b, 0, t)
    host = [[hb.banks[b].numpy().reshape(w.E, -1)] for b in range(len(hb.banks))]
    res = {"workload": name, "format": w.fmt, "hidden": w.H, "inter": w.I, "experts": w.E, "topk": w.k,
           "layers": w.L, "slots": w.S, "bytes_per_expert": bpe,
           "host_bank_GiB": sum(t.numel() for t in hb.banks) / 2**30, "host_bank_gen_s": gen_s,
           "oracle_host": _host_info()}
    log(f"{name}: host banks {res['host_bank_GiB']:.2f} GiB in {gen_s:.1f}s")

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def capture(ids_t, slot_t, y_t=None):
        gm = cache.get_misses()
        gsl = torch.tensor([m[0] for m in gm], dtype=torch.long, device=dev)
        out = {"ids": ids_t.cpu().numpy().copy(), "slot_ids": slot_t.cpu().numpy().copy(), "misses": gm,
               "rows": [cache.slot_bank_view(b)[gsl].cpu().numpy() for b in range(len(hb.banks))]}
        if y_t is not None:
            out["y"] = y_t.view(torch.bfloat16).double().cpu().numpy()
        return out

    # ------------------------------------------------------------ decode step per miss rate
    ctx = {"cache": cache, "bpe": bpe, "hb": hb}
    decode = []
    batches = w.batches if name == "bf16_tiny" else (1,)
    rates = sorted(w.miss_rates)
    if headline:
        rates = [args.miss_rate] + [r for r in rates if abs(r - args.miss_rate) > 1e-12]
    for bs in batches:
        x = synth.activations(bs, w.H, 0, w.name).to(dev)
        wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
        ids = torch.empty((bs, w.k), dtype=torch.int32, device=dev)
        wts = torch.empty((bs, w.k), dtype=torch.float32, device=dev)
        slot_ids = torch.empty_like(ids)
        y = torch.empty((bs, w.H), dtype=torch.int16, device=dev)
        rws = torch.empty(oes.route_workspace_bytes(bs, w.H, w.E), dtype=torch.uint8, device=dev)
        fws = torch.empty(cache.ffn_workspace_bytes(bs, w.k), dtype=torch.uint8, device=dev)
        oes.route(x, wg, w.k, ids, wts, rws)
        torch.cuda.synchronize()
        routed = ids.cpu().numpy()
        active = len(set(routed.ravel().tolist()))
        xb, wgb = x.cpu().numpy().view(np.uint16), wg.cpu().numpy().view(np.uint16)

        def prepare(mr, routed=routed, active=active):
            misses = formulas.num_misses(active, mr)
            owner, stamp, clock, pre = synth.forced_miss_state(w.S, w.E, 0, routed, misses)
            return misses, owner, stamp, clock, pre

        def run_steps(mr, steps, warmup, parts, x=x, wg=wg, ids=ids, wts=wts, slot_ids=slot_ids, y=y, rws=rws,
                      fws=fws, prepare=prepare):
            """Enqueue warmup + steps layer steps back to back, the slot table restored
            on the device between steps (outside the events).  parts=False: events
            only at step boundaries; parts=True: also between route, ensure, copy and
            FFN, for the breakdown."""
            misses, owner, stamp, clock, pre = prepare(mr)
            cache.set_state(owner, stamp, clock)
            if pre:
                cache.load_rows([p[0] for p in pre], [p[1] for p in pre])
            cache.snapshot()
            torch.cuda.synchronize()
            _hold_gpu(0.2 * (warmup + steps))
            rec = []
            for i in range(warmup + steps):
                cache.restore()
                e = [ev() for _ in range(5 if parts else 2)]
                e[0].record(stream)
                oes.route(x, wg, w.k, ids, wts, rws)
                if parts:
                    e[1].record(stream)
                cache.ensure_experts(0, ids, slot_ids)
                if parts:
                    e[2].record(stream)
                cache.copy_missing()
                if parts:
                    e[3].record(stream)
                cache.expert_ffn(x, slot_ids, wts, y, fws)
                e[-1].record(stream)
                if i >= warmup:
                    rec.append(e)
            torch.cuda.synchronize()
            cache.check()
            total = np.array([r[0].elapsed_time(r[-1]) for r in rec])
            if not parts:
                return misses, total, None
            return misses, total, np.array([[r[j].elapsed_time(r[j + 1]) for j in range(4)] for r in rec])

        for mr in rates:
            is_head = headline and bs == 1 and abs(mr - args.miss_rate) < 1e-12
            steps = args.steps if is_head else max(5, args.steps // 3)
            wu = args.warmup if is_head else 2
            if is_head:
                # one untimed pass of the same steps first: the first host-link-heavy pass
                # of a process has run several per cent slow on some boxes (all of its
                # steps, not only the warm-up ones), the passes after it did not
                run_steps(mr, steps, wu, parts=False)
            misses, total, _ = run_steps(mr, steps, wu, parts=False)
            _, ptotal, parts = run_steps(mr, steps, wu, parts=True)
            ms = float(total.mean())
            row = {"what": f"decode bs={bs} mr={mr}", "bs": bs, "miss_rate": mr, "active": active, "misses": misses,
                   "ms_per_step": ms, "ms_median": float(np.median(total)), "steps": int(steps),
                   "tok_ms": ms * w.L, "decode_tok_s": 1000.0 / (w.L * ms),
                   "ms_per_step_with_part_events": float(ptotal.mean()),
                   "route_ms": float(parts[:, 0].mean()), "ensure_ms": float(parts[:, 1].mean()),
                   "copy_ms": float(parts[:, 2].mean()), "ffn_ms": float(parts[:, 3].mean())}
            if misses:
                row["copy_GBps"] = misses * bpe / (row["copy_ms"] * 1e6)
            # every step of the loop starts from the same state: the last one's outputs are the step's
            gpu = capture(ids, slot_ids, y)
            _, owner, stamp, clock, _ = prepare(mr)
            orc, tim = _oracle_step(w, host, (owner, stamp, clock), hb.row_bytes, xb=xb, wgb=wgb)
            row["parity"] = _gate(gpu, orc, tol)
            row["oracle"] = dict(tim, tok_s=1000.0 / (w.L * tim["ms_per_step"]))
            decode.append(row)
            if is_head:
                ctx.update(headline_row=row, x=x, wg=wg, rws=rws, fws=fws, prepare=prepare)
            log(f"{name} decode", _r({k: v for k, v in row.items() if k not in ("parity", "oracle")}),
                "parity", row["parity"]["ok"], "oracle ms", round(tim["ms_per_step"], 1))
    decode.sort(key=lambda r: (r["bs"], r["miss_rate"]))
    res["decode"] = decode

    # ------------------------------------------------------------ copy sweep
    sweep = []
    if not args.no_sweep:
        modes = [("", 1, oes.COPY_ZERO), ("_per_bank", 0, oes.COPY_ZERO)]
        if not args.no_sdma:
            modes.append(("_sdma", 1, oes.COPY_SDMA))
        for bs in w.batches:
            sids = synth.synthetic_ids(bs, w.k, w.E, 0, w.name)
            d_ids = sids.to(dev)
            d_slots = torch.empty_like(d_ids)
            act = formulas.active_unique(bs, w.k, w.E)
            for mr in w.miss_rates:
                m = formulas.num_misses(act, mr)
                owner, stamp, clock, _ = synth.forced_miss_state(w.S, w.E, 0, sids.numpy(), m)
                row = {"what": f"copy bs={bs} mr={mr}", "bs": bs, "active": act, "miss_rate": mr, "misses": m}
                cache.set_state(owner, stamp, clock)
                cache.snapshot()
                for key, fused, mode in modes:
                    cache.set_option(oes.OPT_FUSED_COPY, fused)
                    cache.set_option(oes.OPT_COPY_MODE, mode)
                    marks = []
                    for _ in range(args.repeat):
                        cache.restore()
                        a, b = ev(), ev()
                        a.record(stream)
                        cache.ensure_experts(0, d_ids, d_slots)
                        cache.copy_missing()
                        b.record(stream)
                        marks.append((a, b))
                    torch.cuda.synchronize()
                    tm = statistics.median([a.elapsed_time(b) for a, b in marks])
                    row["time_ms" + key] = tm
                    row["bw_GBps" + key] = formulas.bw_gbps(m, bpe, tm) if m else None
                cache.set_option(oes.OPT_FUSED_COPY, 1)
                cache.set_option(oes.OPT_COPY_MODE, oes.COPY_ZERO)
                row["copy_MiB"] = formulas.copy_mib(m, bpe)
                row["tok_ms"] = formulas.tok_ms(row["time_ms"], w.L)
                if probes and row["bw_GBps"]:
                    row["frac_h2d_peak"] = row["bw_GBps"] / probes["h2d_peak_GBps"]
                gpu = capture(d_ids, d_slots)
                orc, tim = _oracle_step(w, host, (owner, stamp, clock), hb.row_bytes, ids=sids.numpy(), ffn=False)
                row["parity"] = _gate(gpu, orc, routed=False)
                row["oracle"] = tim
                sweep.append(row)
                log(f"{name} sweep", _r({k: v for k, v in row.items() if k not in ("parity", "oracle")}),
                    "parity", row["parity"]["ok"])
        cache.check()
    res["copy_sweep"] = sweep

    # ------------------------------------------------------------ the FFN alone, cold
    res["ffn"] = _ffn_cold(w, cache, hb, host, sc, probes, log)
    return res, ctx


def _ffn_cold(w, cache, hb, host, sc, probes, log, launches=64):
    """The expert FFN alone at bs=1 and at the workload's larger batches, cold.

    The layer-0 host banks are also registered under layers 1..R-1, and the same
    routed tokens are remapped for each of those layers (every slot first owned
    by another layer), so R launches read R disjoint sets of the same experts'
    bytes: back-to-back launches that cycle over them find nothing of the last R-1
    launches' rows in the 256 MB memory-side cache once R * u * bpe exceeds it.
    Bytes per launch = u * bytes_per_expert with u the distinct experts routed."""
    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth
    from oracle import ffn as offn
    from oracle import route as oroute

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    bpe = sc.bytes_per_expert
    out = {}
    for bs in sorted(set((1,) + tuple(w.batches))):
        x = synth.activations(bs, w.H, 0, w.name, step=101).to(dev)
        wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
        xb, wgb = x.cpu().numpy().view(np.uint16), wg.cpu().numpy().view(np.uint16)
        oids, ow, _ = oroute.route(xb, wgb, w.k)
        u = len(set(oids.ravel().tolist()))
        R = max(1, min(16, w.S // u, w.L))
        for layer in range(1, R):
            for b, t in enumerate(hb.banks):
                cache.set_source(b, layer, t)
        owner, stamp, clock = synth.foreign_state(w.S, w.E)
        owner = owner + (w.L - 1) * w.E        # owners of no layer driven here
        cache.set_state(owner, stamp, clock)
        ids = torch.from_numpy(oids).to(dev)
        wts = torch.from_numpy(ow.astype(np.float32)).to(dev)
        maps = []
        for layer in range(R):
            sl = torch.empty_like(ids)
            cache.ensure_experts(layer, ids, sl)
            cache.copy_missing()
            maps.append(sl)
        y = torch.empty((bs, w.H), dtype=torch.int16, device=dev)
        ws = torch.empty(cache.ffn_workspace_bytes(bs, w.k), dtype=torch.uint8, device=dev)
        def timed(path):
            cache.set_option(oes.OPT_FFN_PATH, path)
            for i in range(4):
                cache.expert_ffn(x, maps[i % R], wts, y, ws)
            torch.cuda.synchronize()
            cache.check()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            _hold_gpu(5.0)
            a.record(stream)
            for i in range(launches):
                cache.expert_ffn(x, maps[i % R], wts, y, ws)
            b.record(stream)
            torch.cuda.synchronize()
            cache.check()
            return a.elapsed_time(b) / launches

        # several tokens: both FFN paths beside the default choice (run last, so that y
        # below is the default path's)
        paths = {}
        if bs > 1:
            paths = {"per_pair_ms": timed(oes.FFN_PER_PAIR), "grouped_ms": timed(oes.FFN_GROUPED)}
        ms = timed(oes.FFN_AUTO)
        nbytes = u * bpe
        row = {"what": f"ffn bs={bs}", "bs": bs, "unique_experts": u, "bytes": nbytes, "avg_ms": ms,
               "GBps": nbytes / (ms * 1e6), "frac_of_hbm_peak": nbytes / (ms * 1e6) / HBM_PEAK_GBS,
               "disjoint_sets": R, "launches": launches, **paths,
               "traffic": _pmc_traffic(f"expert_ffn_{w.name}_bs{bs}" if bs > 1 else f"expert_ffn_{w.name}")}
        if probes:
            row["frac_of_measured_hbm_read"] = row["GBps"] / probes["hbm_read_GBps"]
        # the last launch ran on layer (launches - 1) % R's slots: check it against the oracle
        # on two tokens (every token is checked in the tests)
        sel = [0] if bs == 1 else [0, bs - 1]
        m_last = maps[(launches - 1) % R].cpu().numpy()
        own, _, _ = cache.get_state()
        t0 = time.perf_counter()
        ref = offn.expert_ffn(w.fmt, w.H, w.I, xb[sel], m_last[sel], ow[sel].astype(np.float32).astype(np.float64),
                              lambda s: [host[bb][0][int(own[s]) % w.E] for bb in range(len(host))])
        t_ffn = (time.perf_counter() - t0) * 1e3
        err = float(offn.rel_l2(y.view(torch.bfloat16).double().cpu().numpy()[sel], ref))
        row["parity"] = {"ffn_rel_l2": err, "ffn_tol": _tol(w.fmt), "tokens": sel, "ok": err <= _tol(w.fmt)}
        row["oracle"] = {"t_ffn_ms": t_ffn, "tokens": len(sel)}
        out[f"bs{bs}"] = row
        log(f"{w.name} ffn", _r({k: v for k, v in row.items() if k not in ("parity", "oracle")}),
            "parity", row["parity"]["ok"])
    return out


# ============================================================================ prefill
def _prefill(w, probes, log):
    """MXFP4 prefill: grouped FFN time (MFMA), one layer's stream time, the
    overlapped loop, and the oracle gate on the layer FFN restricted to a sample
    of experts (the GPU runs the same restricted FFN: pairs of other experts get
    id -1), whose oracle time scales to the whole layer by the expert count."""
    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth
    from oracle import ffn as offn
    from oracle import route as oroute
    from synth.workloads import make_host_banks

    dev = torch.device("cuda:0")
    t0 = time.time()
    hb = make_host_banks(w)
    gen_s = time.time() - t0
    sc = oes.schema_make(w.fmt, w.stream_layers, w.E, w.H, w.I)
    L = oes.Layers(sc, 2, 0)
    for layer in range(w.stream_layers):
        for b, t in enumerate(hb.banks):
            L.set_source(b, layer, t)   # one host bank reused under every layer id (the tests use distinct ones)
    L.prefetch(0)
    logits = synth.router_logits(w.tokens, w.E, 0, w.name)
    ids = torch.empty((w.tokens, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.tokens, w.k), dtype=torch.float32, device=dev)
    oes.route_logits(logits.to(dev), w.k, ids, wts)
    x = synth.activations(w.tokens, w.H, 0, w.name).to(dev)
    y = torch.empty((w.tokens, w.H), dtype=torch.int16, device=dev)
    ws = torch.empty(L.ffn_workspace_bytes(w.tokens, w.k), dtype=torch.uint8, device=dev)
    for _ in range(3):
        L.ffn(0, x, ids, wts, y, ws)
    marks = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        L.ffn(0, x, ids, wts, y, ws)
        b.record()
        marks.append((a, b))
    torch.cuda.synchronize()
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in marks]))
    flops = 6.0 * w.tokens * w.k * w.H * w.I
    wbytes = w.E * sc.bytes_per_expert
    cs = torch.cuda.Stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(cs)
    L.prefetch(1, cs)
    b.record(cs)
    b.synchronize()
    copy_ms = a.elapsed_time(b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    L.prefetch(0, cs)
    for layer in range(w.stream_layers):
        if layer + 1 < w.stream_layers:
            L.prefetch(layer + 1, cs)
        L.ffn(layer, x, ids, wts, y, ws)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0

    # the gate: routed ids, then the FFN restricted to 8 experts, against the oracle
    oids, ow = oroute.topk_softmax(logits.numpy(), w.k)
    ids_ok = bool(np.array_equal(ids.cpu().numpy(), oids))
    chosen = np.arange(0, w.E, w.E // 8)[:8]
    sub = np.where(np.isin(oids, chosen), oids, -1).astype(np.int32)
    L.ffn(w.stream_layers - 1, x, torch.from_numpy(sub).to(dev), wts, y, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ref = offn.expert_ffn(w.fmt, w.H, w.I, x.cpu().numpy().view(np.uint16), sub,
                          ow.astype(np.float32).astype(np.float64),
                          lambda e: [hb.row(bb, e).numpy() for bb in range(len(hb.banks))])
    t_sample = (time.perf_counter() - t1) * 1e3
    err = float(offn.rel_l2(y.view(torch.bfloat16).double().cpu().numpy(), ref))
    tol = _tol(w.fmt)
    gate = {"what": "prefill layer (8 experts)", "parity": {"ids": ids_ok, "ffn_rel_l2": err, "ffn_tol": tol,
                                                             "experts": chosen.tolist(),
                                                             "ok": ids_ok and err <= tol},
            "oracle": {"t_ffn_sample_ms": t_sample, "pairs": int((sub >= 0).sum()),
                       "t_layer_est_ms": t_sample * w.E / len(chosen),
                       "sample": f"the layer FFN restricted to experts {chosen.tolist()} "
                                 f"({int((sub >= 0).sum())} of {w.tokens * w.k} pairs); the layer estimate "
                                 f"scales it by {w.E}/{len(chosen)}",
                       "host": _host_info()}}
    out = {"workload": w.name, "tokens": w.tokens, "flops": flops, "ffn_ms": ffn_ms,
           "ffn_TFLOPs": flops / (ffn_ms * 1e9), "ffn_weight_GBps": wbytes / (ffn_ms * 1e6),
           "layer_bytes": wbytes, "bytes_per_expert": sc.bytes_per_expert, "layer_copy_ms": copy_ms,
           "stream_GBps": wbytes / (copy_ms * 1e6), "layers": w.stream_layers,
           "overlapped_ms_per_layer": wall_ms / w.stream_layers, "host_bank_gen_s": gen_s,
           "instruction": "v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e2m1), two per product", "gate": gate}
    if probes:
        out["stream_frac_of_measured_h2d_peak"] = out["stream_GBps"] / probes["h2d_peak_GBps"]
    log("prefill", _r({k: v for k, v in out.items() if k != "gate"}), "parity", gate["parity"])
    L.close()
    return out


def _cpu_baseline(w, hb, x, wg, mr, budget_s):
    """The oracle, as it stands, on this host: route + LRU + row copies + FFN for bs=1
    steps of the headline workload from the headline's forced-miss state, repeated
    within `budget_s` (at most 25), median."""
    import numpy as np

    import synth
    from oracle import formulas
    from oracle import route as oroute

    xb = x.cpu().numpy().view(np.uint16)
    wgb = wg.cpu().numpy().view(np.uint16)
    host = [[hb.banks[b].numpy().reshape(w.E, -1)] for b in range(len(hb.banks))]
    ids, _, _ = oroute.route(xb, wgb, w.k)
    active = len(set(ids.ravel().tolist()))
    owner, stamp, clock, _ = synth.forced_miss_state(w.S, w.E, 0, ids, formulas.num_misses(active, mr))
    times, parts = [], []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 25):
        _, tim = _oracle_step(w, host, (owner, stamp, clock), hb.row_bytes, xb=xb, wgb=wgb)
        times.append(tim["ms_per_step"])
        parts.append(tim)
    ms = float(np.median(times))
    info = _host_info()
    return {"value": 1000.0 / (w.L * ms), "unit": "tok/s", "cores": info["blas_threads"], "kind": "oracle",
            "ms_per_step": ms, "sample": f"{len(times)} bs=1 decode steps of {w.name} at miss_rate {mr} "
                                        f"(route, LRU, row copies, float64 FFN), median",
            "parts_ms": {k: float(np.median([p[k] for p in parts])) for k in parts[0]},
            "cpu_model": info["cpu_model"], "cpu_count": info["cpu_count"], "affinity": info["affinity"]}


def _hybrid(cache, hb, w, bpe, x, wg, rws, fws, prepare, probes, per_mr, args, log):
    """The hybrid backend on the bench workload (benchmark guide §5.2-§5.4).

    ft bench bw: the DRAM read ceiling (every host bank byte read once by the
    executor's threads) beside the pinned H2D ceiling; the real kernels - the
    CPU executor on k experts of one token (every pair left to the CPU) and the
    PCIe gather of k misses - alone, then overlapped (the gather of k experts
    enqueued, the executor run on k others meanwhile); the decision (alone
    bandwidths) and the fetch fraction (overlapped ones).

    Then the decode layer step at bs=1 and the headline miss rate, hybrid
    (route, then oes_hybrid_step with that fraction) and offload (route,
    ensure, copy, FFN), both timed by wall clock from the route launch to y on
    the host side of a stream sync, since the hybrid step itself waits for the
    remap; the slot table is restored (untimed) before every step.
    """
    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
    cpu = oes.CpuMoe(sc, 0)
    for b, t in enumerate(hb.banks):
        cpu.set_source(b, 0, t)
    out = {"threads": cpu.threads, "format": w.fmt}

    # ceilings
    host_bytes = sum(t.numel() for t in hb.banks)
    reads = [cpu.probe_read(t, t.numel()) for t in hb.banks for _ in range(3)]
    per_bank = [min(reads[3 * b:3 * b + 3]) for b in range(len(hb.banks))]
    out["dram_read_GBps"] = host_bytes / (sum(per_bank) * 1e6)
    out["h2d_GBps"] = probes.get("h2d_peak_GBps") if probes else None

    # real kernels, alone: k experts per call, rotating over E / k disjoint sets
    k, E = w.k, w.E
    sets = [np.arange(i * k, (i + 1) * k, dtype=np.int32).reshape(1, k) for i in range(E // k)]
    xh = synth.activations(1, w.H, 0, w.name)
    allcpu = np.full((1, k), -1, dtype=np.int32)
    wk = np.full((1, k), 1.0 / k, dtype=np.float32)
    yc = np.zeros((1, w.H), dtype=np.float32)
    for i in range(3):
        cpu.run(0, xh, sets[i], allcpu, wk, yc)
    times = []
    for i in range(12):
        t0 = time.perf_counter()
        cpu.run(0, xh, sets[(3 + i) % len(sets)], allcpu, wk, yc)
        times.append(time.perf_counter() - t0)
    cpu_ms = float(np.median(times)) * 1e3
    out["cpu_moe_ms"] = cpu_ms
    out["cpu_moe_GBps"] = k * bpe / (cpu_ms * 1e6)
    full = [r for r in per_mr if r["miss_rate"] == 1.0 and r.get("copy_GBps")]
    out["pcie_gather_GBps"] = full[0]["copy_GBps"] if full else None

    # overlapped: the gather of k misses (every slot foreign) with the executor on k other experts
    owner, stamp, clock = synth.foreign_state(w.S, w.E)
    d_ids = [torch.from_numpy(sets[i]).to(dev) for i in range(len(sets))]
    d_slots = torch.empty((1, k), dtype=torch.int32, device=dev)
    gpu_ms, cpu_ov = [], []
    for i in range(8):
        cache.set_state(owner, stamp, clock)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cache.ensure_experts(0, d_ids[i % len(sets)], d_slots)
        cache.copy_missing()
        b.record(stream)
        t0 = time.perf_counter()
        cpu.run(0, xh, sets[(i + len(sets) // 2) % len(sets)], allcpu, wk, yc)
        cpu_ov.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        gpu_ms.append(a.elapsed_time(b))
    cache.check()
    out["overlap_cpu_GBps"] = k * bpe / (float(np.median(cpu_ov)) * 1e9)
    out["overlap_pcie_GBps"] = k * bpe / (float(np.median(gpu_ms)) * 1e6)
    pcie = out["pcie_gather_GBps"] or out["overlap_pcie_GBps"]
    use, _ = oes.hybrid_decide(w.fmt, out["cpu_moe_GBps"], pcie)
    _, frac = oes.hybrid_decide(w.fmt, out["overlap_cpu_GBps"], out["overlap_pcie_GBps"])
    out["decision"] = "hybrid" if use else "offload"
    out["fetch_fraction"] = frac

    # the decode layer step, hybrid vs offload, wall clock with a sync per step
    mr = args.miss_rate
    misses, owner, stamp, clock, pre = prepare(mr)
    cache.set_state(owner, stamp, clock)
    if pre:
        cache.load_rows([p[0] for p in pre], [p[1] for p in pre])
    cache.snapshot()
    x1 = x[:1]
    ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, k), dtype=torch.float32, device=dev)
    slot_ids = torch.empty_like(ids)
    y = torch.empty((1, w.H), dtype=torch.int16, device=dev)
    hws, dws = cache.hybrid_workspace(1, k)
    host_ws = torch.empty(hws, dtype=torch.uint8, pin_memory=True)
    dev_ws = torch.empty(dws, dtype=torch.uint8, device=dev)

    def step(kind):
        cache.restore()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        oes.route(x1, wg, k, ids, wts, rws)
        if kind == "hybrid":
            cache.hybrid_step(cpu, 0, x1, ids, wts, slot_ids, y, fws, host_ws, dev_ws, -1, frac)
        else:
            cache.ensure_experts(0, ids, slot_ids)
            cache.copy_missing()
            cache.expert_ffn(x1, slot_ids, wts, y, fws)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    res = {}
    for kind in ("offload", "hybrid"):
        for _ in range(3):
            step(kind)
        ts = [step(kind) for _ in range(args.hybrid_steps)]
        ms = float(np.median(ts)) * 1e3
        res[kind] = {"ms_per_step": ms, "decode_tok_s": 1000.0 / (w.L * ms)}
    cache.check()
    st = cache.stats()
    res["hybrid"]["fetched_last_step"] = st["last_indices"]
    res["hybrid"]["cpu_experts_last_step"] = st["last_missing_full"] - st["last_indices"]
    out.update({"miss_rate": mr, "misses": misses, "step": res,
                "hybrid_speedup": res["offload"]["ms_per_step"] / res["hybrid"]["ms_per_step"]})
    log("hybrid", {kk: (round(v, 4) if isinstance(v, float) else v) for kk, v in out.items() if kk != "step"}, res)
    cpu.close()
    return out


def _cpu_formats(workloads, pcie_gbps, log, experts=8, repeats=12):
    """ft bench bw per format (benchmark guide §5.2): the CPU executor on `experts`
    experts of one token (banks of 2 * experts experts, rotating over the two
    halves) against that format's measured PCIe gather (pcie_gbps[name], the
    fused gather of its copy sweep); the decision and the fetch fraction.  Block fp8 has no CPU path and stays offload."""
    import numpy as np

    import offloaded_expert_slot_amd as oes
    import synth
    from synth.workloads import Workload, make_host_banks

    out = {}
    for name in ("bf16_h2048", "nvfp4_h7168", "q4_0_h2048", "fp8_h4096"):
        w0 = workloads[name]
        pcie = pcie_gbps.get(name)
        if pcie is None:
            continue
        row = {"format": w0.fmt, "pcie_gather_GBps": pcie}
        if w0.fmt == "fp8_block128":
            use, frac = oes.hybrid_decide(w0.fmt, 0.0, pcie)
            row.update(cpu_moe_GBps=None, decision="hybrid" if use else "offload", fetch_fraction=frac)
            out[name] = row
            continue
        E = 2 * experts
        w = Workload(w0.name, w0.fmt, L=1, E=E, k=experts, H=w0.H, I=w0.I, S=E)
        hb = make_host_banks(w)
        sc = oes.schema_make(w.fmt, 1, E, w.H, w.I)
        cpu = oes.CpuMoe(sc, 0)
        for b, t in enumerate(hb.banks):
            cpu.set_source(b, 0, t)
        xh = synth.activations(1, w.H, 0, w.name)
        sets = [np.arange(h * experts, (h + 1) * experts, dtype=np.int32).reshape(1, experts) for h in range(2)]
        allcpu = np.full((1, experts), -1, dtype=np.int32)
        wk = np.full((1, experts), 1.0 / experts, dtype=np.float32)
        yc = np.zeros((1, w.H), dtype=np.float32)
        for i in range(2):
            cpu.run(0, xh, sets[i], allcpu, wk, yc)
        ts = []
        for i in range(repeats):
            t0 = time.perf_counter()
            cpu.run(0, xh, sets[i % 2], allcpu, wk, yc)
            ts.append(time.perf_counter() - t0)
        ms = float(np.median(ts)) * 1e3
        gbps = experts * sc.bytes_per_expert / (ms * 1e6)
        use, frac = oes.hybrid_decide(w.fmt, gbps, pcie)
        row.update(cpu_moe_ms=ms, cpu_moe_GBps=gbps, decision="hybrid" if use else "offload", fetch_fraction=frac)
        out[name] = row
        log("cpu format", {k: (round(v, 4) if isinstance(v, float) else v) for k, v in row.items()})
        cpu.close()
        del hb
    return out


def _resize(cache, w, bpe, log):
    """Slot-pool resize on the bench cache (host-synchronous calls, wall clock):
    shrink to half the slots, then grow back.  Each call moves half the slots'
    rows (every kept slot, bpe bytes each) device to device, besides allocating
    the new banks and table and freeing the old ones."""
    import torch

    torch.cuda.synchronize()
    half = w.S // 2
    t0 = time.perf_counter()
    cache.resize(half)
    t1 = time.perf_counter()
    cache.resize(w.S)
    t2 = time.perf_counter()
    moved = half * bpe
    out = {"slots": w.S, "shrunk_to": half, "moved_bytes": moved, "shrink_ms": (t1 - t0) * 1e3,
           "grow_ms": (t2 - t1) * 1e3, "shrink_GBps": moved / ((t1 - t0) * 1e9),
           "grow_GBps": moved / ((t2 - t1) * 1e9)}
    log("resize", {k: (round(v, 3) if isinstance(v, float) else v) for k, v in out.items()})
    return out


def _pmc_traffic(kernel):
    """HBM bytes per launch of `kernel` from the FETCH_SIZE / WRITE_SIZE passes
    summarised under profiles/, or None once the kernel's source has changed
    since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            f = line.split()
            if len(f) == 5 and f[0] == "traffic" and f[1] == kernel:
                kv = dict(x.split("=", 1) for x in f[2:])
                src = os.path.join(ROOT, kv["source"])
                if os.path.exists(src) and hashlib.sha256(open(src, "rb").read()).hexdigest() == kv["sha256"]:
                    return int(kv["bytes_per_launch"])
                return None
    return None



_HOLD = {}


def _hold_gpu(ms):
    """Keep the current stream busy for about `ms` milliseconds with a spinning
    kernel, so that the host enqueues the timed launches that follow before the
    GPU reaches them: the events then time the GPU work alone, not the host's
    launch rate (which can be the slower of the two for microsecond kernels).
    The spin itself lies before the first event."""
    import torch
    if "cycles_per_ms" not in _HOLD:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1 << 20)
        b.record()
        b.synchronize()
        _HOLD["cycles_per_ms"] = (1 << 20) / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_HOLD["cycles_per_ms"] * ms))


if __name__ == "__main__":
    main()
