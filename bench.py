"""Benchmark of the per-layer offloaded-expert MoE step on one MI355X.

Metric: copy_missing GB/s + tok_ms per miss rate; MoE-layer decode tok/s at bs=1.

Workload (default): bf16 banks, H=2048, I=768, E=128 experts, top-8, L=48
MoE layers, a 1024-slot pool whose every slot starts owned by another layer;
layer 0 is driven and per-token costs are extrapolated over L layers (FreeToken
MoE benchmark guide §4.3-§4.4).  Inputs are seeded synthetic tensors resident
in HBM (activations, router) and in pinned host banks (experts).

One "step" = route -> ensure_experts -> copy_missing -> expert_ffn for one
token (bs=1), with the slot table restored on the device (untimed) before each
step so that misses = round(active * miss_rate) of the routed experts miss.
Steps are enqueued back to back and each is timed with HIP events on the
launch stream at its two ends; value = 1000 / (L * ms_per_step).  A second pass
with events between the four parts gives the breakdown and the copy's time.

Also printed (same JSON line): the copy sweep of the benchmark guide's columns
(bs, active, miss_rate, misses, time_ms, copy_MiB, bw_GBps, tok_ms; median of
25 event-timed ensure+copy repeats, fused and per-bank), decode tok/s at every
miss rate, the measured ceilings (pinned H2D by DMA and by the zero-copy
kernel, HBM streaming read, the bf16 and the block-scaled e4m3 x e2m1 MFMA
loops), the roofline of the dominant kernel and of the FFN, copy_missing of
every decode bank format (8 misses), the hybrid backend (host DRAM read and
link ceilings, the CPU MoE executor and the PCIe gather alone and overlapped,
the decision and fetch split, the hybrid decode layer step beside the offload
one), the cold decode FFN of every decode bank format (bf16, fp8 block, nvfp4,
GGUF Q4_0) at its workload's shape, a slot-pool resize (half the slots and
back), the MXFP4 prefill layer (grouped FFN on the block-scaled MFMA,
whole-layer stream, the overlapped loop over 4 layers) and the CPU oracle timed
on this host.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bf16_h2048")
    ap.add_argument("--miss-rate", type=float, default=0.5)
    ap.add_argument("--repeat", type=int, default=25, help="repeats per copy-sweep row (median)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill (MXFP4 layer stream) part")
    ap.add_argument("--no-hybrid", action="store_true", help="skip the hybrid backend (CPU executor) part")
    ap.add_argument("--hybrid-steps", type=int, default=20, help="timed hybrid / synced offload layer steps")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the step has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth
    from synth.workloads import WORKLOADS, make_host_banks

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    t0 = time.time()
    hb = make_host_banks(w)
    log(f"host banks ready ({sum(b.numel() for b in hb.banks) / 2**30:.2f} GiB pinned) in {time.time() - t0:.1f}s")
    sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
    bpe = sc.bytes_per_expert
    cache = oes.Cache(sc, w.S, 0)
    for b, t in enumerate(hb.banks):
        cache.set_source(b, 0, t)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---------------------------------------------------------------- ceilings
    probes = {}
    if not args.no_probes:
        src = hb.banks[0]
        nbytes = (src.numel() // 16) * 16
        dbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dma = [oes.probe_h2d_dma(dbuf, src, nbytes) for _ in range(5)]
        zc = [oes.probe_h2d_kernel(dbuf, src, nbytes, 1024) for _ in range(5)]
        big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        big.fill_(1)
        sink = torch.zeros(4, dtype=torch.float32, device=dev)
        hbm = [oes.probe_hbm_read(big, big.numel(), sink) for _ in range(5)]
        mfma = [oes.probe_mfma_bf16(2048, 10000, sink) for _ in range(3)]
        mfma_f8f4 = [oes.probe_mfma_f8f4(2048, 5000, sink) for _ in range(3)]
        # streaming reads of the FFN's byte count, back to back over 16 distinct
        # regions (1.2 GB), timed like the FFN alone below
        fb = (w.k * bpe // 16) * 16
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
        del big, dbuf
        log("probes", {k: round(v, 1) for k, v in probes.items()})

    # ---------------------------------------------------------------- decode step at bs=1
    n = 1
    x = synth.activations(n, w.H, 0, w.name).to(dev)
    wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
    ids = torch.empty((n, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((n, w.k), dtype=torch.float32, device=dev)
    slot_ids = torch.empty_like(ids)
    y = torch.empty((n, w.H), dtype=torch.int16, device=dev)
    rws = torch.empty(oes.route_workspace_bytes(n, w.H, w.E), dtype=torch.uint8, device=dev)
    fws = torch.empty(cache.ffn_workspace_bytes(n, w.k), dtype=torch.uint8, device=dev)
    oes.route(x, wg, w.k, ids, wts, rws)
    torch.cuda.synchronize()
    routed = ids.cpu().numpy()
    active = len(set(routed.ravel().tolist()))
    u_bytes = active * bpe

    def prepare(mr):
        misses = int(round(active * mr))
        owner, stamp, clock, pre = synth.forced_miss_state(w.S, w.E, 0, routed, misses)
        return misses, owner, stamp, clock, pre

    def run_steps(mr, steps, warmup, parts):
        """Enqueue warmup + steps layer steps back to back, the slot table restored
        on the device between steps (outside the events).  parts=False: events
        only at step boundaries (each event recorded inside a step idles the GPU
        for several microseconds); parts=True: also between route, ensure, copy
        and FFN, for the breakdown."""
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

    per_mr = []
    headline = None
    gpu_step = None
    # the headline miss rate runs first, so that its copy launches are the first
    # gather dispatches of the run: 0..W+K-1 the timed pass, W+K..2(W+K)-1 the
    # breakdown pass (the profile summary averages the latter's timed ones)
    rates = [args.miss_rate] + [r for r in sorted(w.miss_rates) if abs(r - args.miss_rate) > 1e-12]
    for mr in rates:
        is_head = abs(mr - args.miss_rate) < 1e-12
        steps = args.steps if is_head else max(5, args.steps // 3)
        wu = args.warmup if is_head else 2
        misses, total, _ = run_steps(mr, steps, wu, parts=False)
        _, ptotal, parts = run_steps(mr, steps, wu, parts=True)
        ms = float(total.mean())
        row = {"miss_rate": mr, "misses": misses, "ms_per_step": ms, "ms_median": float(np.median(total)),
               "tok_ms": ms * w.L, "decode_tok_s": 1000.0 / (w.L * ms),
               "ms_per_step_with_part_events": float(ptotal.mean()),
               "route_ms": float(parts[:, 0].mean()), "ensure_ms": float(parts[:, 1].mean()),
               "copy_ms": float(parts[:, 2].mean()), "ffn_ms": float(parts[:, 3].mean())}
        if misses:
            row["copy_GBps"] = misses * bpe / (row["copy_ms"] * 1e6)
        per_mr.append(row)
        per_mr.sort(key=lambda r: r["miss_rate"])
        if is_head:
            headline = (row, total, parts)
            # the step's outputs (every step of the loop starts from the same state)
            gm = cache.get_misses()
            gslots = torch.tensor([m[0] for m in gm], dtype=torch.long, device=dev)
            gpu_step = {"ids": ids.cpu().numpy().copy(), "slot_ids": slot_ids.cpu().numpy().copy(),
                        "y": y.view(torch.bfloat16).double().cpu().numpy(), "misses": gm,
                        "rows": [cache.slot_bank_view(b)[gslots].cpu().numpy() for b in range(len(hb.banks))]}
        log("decode", {k: (round(v, 4) if isinstance(v, float) else v) for k, v in row.items()})

    # FFN alone (HBM roofline): back-to-back launches, each on one of 16 slot maps
    # of 8 distinct slots (128 slots, 1.2 GB in all), so that no launch finds its
    # rows in the 256 MB memory-side cache from the previous ones, as in a real
    # token where every layer has other experts.  Slot contents do not matter for
    # the time; the step loop above keeps its own state.
    rng = np.random.default_rng(0)
    nsets = max(1, min(16, w.S // w.k))   # disjoint slot maps the pool holds (16 for the bench workload)
    pool = rng.permutation(w.S)[: nsets * w.k]
    maps = [torch.from_numpy(pool[i * w.k:(i + 1) * w.k].astype(np.int32).reshape(1, w.k)).to(dev)
            for i in range(nsets)]
    for i in range(4):
        cache.expert_ffn(x, maps[i], wts, y, fws)
    a, b = ev(), ev()
    n_ffn = 64
    torch.cuda.synchronize()
    _hold_gpu(5.0)
    a.record(stream)
    for i in range(n_ffn):
        cache.expert_ffn(x, maps[i % nsets], wts, y, fws)
    b.record(stream)
    torch.cuda.synchronize()
    cache.check()
    ffn_alone_ms = a.elapsed_time(b) / n_ffn
    ffn_bytes = w.k * bpe
    log("ffn", {"launches": n_ffn, "slot_maps": nsets, "ms_per_launch": round(ffn_alone_ms, 5)})

    ffn_formats = _ffn_formats(WORKLOADS, 16, n_ffn, probes, log)
    copy_formats = _copy_formats(WORKLOADS, probes, log)

    # ---------------------------------------------------------------- copy sweep
    sweep = []
    if not args.no_sweep:
        for bs in w.batches:
            sids = synth.synthetic_ids(bs, w.k, w.E, 0, w.name)
            d_ids = sids.to(dev)
            d_slots = torch.empty_like(d_ids)
            act = min(w.E, bs * w.k)
            for mr in w.miss_rates:
                m = int(round(act * mr))
                owner, stamp, clock, _ = synth.forced_miss_state(w.S, w.E, 0, sids.numpy(), m)
                row = {"bs": bs, "active": act, "miss_rate": mr, "misses": m}
                cache.set_state(owner, stamp, clock)
                cache.snapshot()
                for fused in (1, 0):
                    cache.set_option(oes.OPT_FUSED_COPY, fused)
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
                    key = "" if fused else "_per_bank"
                    row["time_ms" + key] = tm
                    row["bw_GBps" + key] = (m * bpe / (tm * 1e6)) if m else None
                row["copy_MiB"] = m * bpe / 2**20
                row["tok_ms"] = row["time_ms"] * w.L
                if probes and row["bw_GBps"]:
                    row["frac_h2d_peak"] = row["bw_GBps"] / probes["h2d_peak_GBps"]
                sweep.append(row)
                log("sweep", {k: (round(v, 4) if isinstance(v, float) else v) for k, v in row.items()})
        cache.set_option(oes.OPT_FUSED_COPY, 1)
        cache.check()

    # ---------------------------------------------------------------- hybrid backend (ft bench bw + the hybrid step)
    hybrid = None
    if not args.no_hybrid:
        hybrid = _hybrid(cache, hb, w, bpe, x, wg, rws, fws, prepare, probes, per_mr, args, log)
        hybrid["formats"] = _cpu_formats(WORKLOADS, copy_formats, log)

    # ---------------------------------------------------------------- slot-pool resize
    resize = _resize(cache, w, bpe, log)

    # ---------------------------------------------------------------- rooflines
    head, total, parts = headline
    ffn_gbs = ffn_bytes / (ffn_alone_ms * 1e6)
    kernels = {
        "expert_ffn": {"bound": "hbm", "achieved": ffn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": ffn_gbs / HBM_PEAK_GBS, "bytes_per_launch": ffn_bytes,
                       "avg_ms": ffn_alone_ms, "traffic": _pmc_traffic("expert_ffn")},
    }
    if probes:
        kernels["expert_ffn"]["frac_of_measured_hbm_read"] = ffn_gbs / probes["hbm_read_GBps"]
        kernels["expert_ffn"]["frac_of_hbm_read_same_bytes"] = ffn_gbs / probes["hbm_read_ffn_bytes_GBps"]
    if head["misses"]:
        cbytes = head["misses"] * bpe
        cgbs = cbytes / (head["copy_ms"] * 1e6)
        kernels["copy_missing"] = {"bound": "host_link", "achieved": cgbs, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                                   "frac": cgbs / PCIE_PEAK_GBS, "bytes_per_launch": cbytes,
                                   "avg_ms": head["copy_ms"], "traffic": _pmc_traffic("copy_missing")}
        if probes:
            kernels["copy_missing"]["frac_of_measured_h2d_peak"] = cgbs / probes["h2d_peak_GBps"]
    dominant = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    roof = dict(kernels[dominant])
    roof = {"kernel": dominant, "bound": roof["bound"], "achieved": roof["achieved"], "peak": roof["peak"],
            "unit": roof["unit"], "frac": roof["frac"], "traffic": roof["traffic"]}

    # ---------------------------------------------------------------- prefill (MXFP4 layer stream)
    prefill = None
    if not args.no_prefill:
        prefill = _prefill(WORKLOADS["mxfp4_prefill"], log)
        kernels["prefill_ffn"] = {"bound": "mfma", "achieved": prefill["ffn_TFLOPs"], "peak": BF16_MFMA_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": prefill["ffn_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS,
                                  "flops_per_launch": prefill["flops"], "avg_ms": prefill["ffn_ms"],
                                  "hbm_GBps": prefill["ffn_weight_GBps"], "traffic": _pmc_traffic("prefill_ffn")}
        # the min(MFMA, HBM x intensity) roofline: 407.7 GFLOP over 1.694 GB of weights
        ridge = min(BF16_MFMA_PEAK_TFLOPS, HBM_PEAK_GBS * prefill["flops"] / prefill["layer_bytes"] / 1e3)
        kernels["prefill_ffn"]["min_roofline_TFLOPs"] = ridge
        kernels["prefill_ffn"]["frac_of_min_roofline"] = prefill["ffn_TFLOPs"] / ridge
        # each bf16 x fp4 product runs as two e4m3 x e2m1 block-scaled MFMAs (the
        # activation's hi and lo planes), which issue at twice the bf16 rate: the
        # measured ceiling of the product is half the f8f4 loop's issued rate
        kernels["prefill_ffn"]["instruction"] = "v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e2m1), two per product"
        if probes:
            kernels["prefill_ffn"]["measured_mfma_ceiling_TFLOPs"] = probes["mfma_f8f4_TFLOPs"] / 2.0
            kernels["prefill_ffn"]["frac_of_measured_mfma_peak"] = prefill["ffn_TFLOPs"] / (probes["mfma_f8f4_TFLOPs"] / 2.0)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(w, hb, x, wg, args.miss_rate, args.cpu_seconds, gpu_step)
        if cpu["parity"] is not None and not cpu["parity"]["ok"]:
            log("PARITY FAILED: the GPU step differs from the oracle", cpu["parity"])
        log("cpu_baseline", cpu)

    ms = head["ms_per_step"]
    out = {
        "metric": METRIC, "value": 1000.0 / (w.L * ms), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "format": w.fmt, "hidden": w.H, "inter": w.I, "experts": w.E,
                   "topk": w.k, "layers": w.L, "slots": w.S, "bs": 1, "miss_rate": args.miss_rate,
                   "misses": head["misses"], "active": active, "bytes_per_expert": bpe},
        "tok_ms": head["tok_ms"], "copy_GBps": head.get("copy_GBps"),
        "roofline": roof, "kernels": kernels, "probes": probes, "decode_per_miss_rate": per_mr,
        "copy_sweep": sweep, "ffn_formats": ffn_formats, "copy_formats": copy_formats, "hybrid": hybrid, "resize": resize, "prefill": prefill,
        "cpu_baseline": cpu, "parity": cpu["parity"] if cpu else None,
    }
    parity_failed = bool(cpu and cpu["parity"] is not None and not cpu["parity"]["ok"])
    if parity_failed:
        # a number from a step that does not match the oracle is not reported
        out["value"] = None
        out["invalid"] = "the headline step differs from the oracle (see parity)"
    print(json.dumps(out), flush=True)
    if parity_failed:
        sys.exit(1)
    cache.close()


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


def _cpu_formats(workloads, copy_formats, log, experts=8, repeats=12):
    """ft bench bw per format (benchmark guide §5.2): the CPU executor on `experts`
    experts of one token (banks of 2 * experts experts, rotating over the two
    halves) against that format's measured PCIe gather; the decision and the
    fetch fraction.  Block fp8 has no CPU path and stays offload."""
    import numpy as np

    import offloaded_expert_slot_amd as oes
    import synth
    from synth.workloads import Workload, make_host_banks

    out = {}
    for name in ("bf16_h2048", "nvfp4_h7168", "q4_0_h2048", "fp8_h4096"):
        w0 = workloads[name]
        pcie = copy_formats[name]["GBps"]
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


def _copy_formats(workloads, probes, log, misses=8, repeats=10):
    """copy_missing of every decode bank format at its workload's shape: `misses`
    experts of layer 0 missing from a pool whose slots all belong to other layers
    (benchmark guide §4.3), median of `repeats` (table restored before each, untimed).
    The banks hold 2 * misses experts: the copy of a row does not depend on E."""
    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth
    from synth.workloads import Workload, make_host_banks

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    for name in ("bf16_h2048", "fp8_h4096", "nvfp4_h7168", "q4_0_h2048"):
        w0 = workloads[name]
        E = 2 * misses
        w = Workload(w0.name, w0.fmt, L=w0.L, E=E, k=misses, H=w0.H, I=w0.I, S=E)
        hb = make_host_banks(w)
        sc = oes.schema_make(w.fmt, w.L, E, w.H, w.I)
        c = oes.Cache(sc, E, 0)
        for b, t in enumerate(hb.banks):
            c.set_source(b, 0, t)
        owner, stamp, clock = synth.foreign_state(E, E)
        c.set_state(owner, stamp, clock)
        c.snapshot()
        ids = torch.arange(misses, dtype=torch.int32, device=dev).reshape(1, misses)
        slots = torch.empty_like(ids)
        marks = []
        for i in range(repeats + 2):
            c.restore()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c.ensure_experts(0, ids, slots)
            a.record(stream)
            c.copy_missing()
            b.record(stream)
            if i >= 2:
                marks.append((a, b))
        torch.cuda.synchronize()
        c.check()
        ms = float(np.median([a.elapsed_time(b) for a, b in marks]))
        nbytes = misses * sc.bytes_per_expert
        row = {"format": w.fmt, "bytes_per_expert": sc.bytes_per_expert, "misses": misses, "copy_ms": ms,
               "GBps": nbytes / (ms * 1e6)}
        if probes:
            row["frac_of_measured_h2d_peak"] = row["GBps"] / probes["h2d_peak_GBps"]
        out[name] = row
        log("copy format", {k: (round(v, 4) if isinstance(v, float) else v) for k, v in row.items()})
        c.close()
        del hb
    torch.cuda.empty_cache()
    return out


def _ffn_formats(workloads, nsets, launches, probes, log):
    """Decode FFN (bs=1, top-k) of every decode bank format at its workload's
    shape, timed cold like the headline's: back-to-back launches over `nsets`
    slot maps of k distinct slots each.  Slot bytes are a constant fill (finite
    values of every element type); they do not change the time."""
    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    for name in ("bf16_h2048", "fp8_h4096", "nvfp4_h7168", "q4_0_h2048"):
        w = workloads[name]
        sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
        slots = nsets * w.k
        c = oes.Cache(sc, slots, 0)
        c.fill_slots(0x11)
        x = synth.activations(1, w.H, 0, w.name).to(dev)
        wts = torch.full((1, w.k), 1.0 / w.k, dtype=torch.float32, device=dev)
        y = torch.empty((1, w.H), dtype=torch.int16, device=dev)
        ws = torch.empty(c.ffn_workspace_bytes(1, w.k), dtype=torch.uint8, device=dev)
        perm = np.random.default_rng(1).permutation(slots).astype(np.int32)
        maps = [torch.from_numpy(perm[i * w.k:(i + 1) * w.k].reshape(1, w.k).copy()).to(dev) for i in range(nsets)]
        for i in range(4):
            c.expert_ffn(x, maps[i], wts, y, ws)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        _hold_gpu(5.0)
        a.record(stream)
        for i in range(launches):
            c.expert_ffn(x, maps[i % nsets], wts, y, ws)
        b.record(stream)
        torch.cuda.synchronize()
        c.check()
        ms = a.elapsed_time(b) / launches
        nbytes = w.k * sc.bytes_per_expert
        row = {"format": w.fmt, "hidden": w.H, "inter": w.I, "topk": w.k, "bytes_per_launch": nbytes,
               "avg_ms": ms, "GBps": nbytes / (ms * 1e6), "frac_of_hbm_peak": nbytes / (ms * 1e6) / HBM_PEAK_GBS}
        if probes:
            row["frac_of_measured_hbm_read"] = row["GBps"] / probes["hbm_read_GBps"]
        out[name] = row
        log("ffn format", {k: (round(v, 4) if isinstance(v, float) else v) for k, v in row.items()})
        c.close()
        del x, y, ws, maps
    torch.cuda.empty_cache()
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


def _prefill(w, log):
    """MXFP4 prefill: grouped FFN time (MFMA), one layer's stream time, and the overlapped loop."""
    import numpy as np
    import torch

    import offloaded_expert_slot_amd as oes
    import synth
    from synth.workloads import make_host_banks

    dev = torch.device("cuda:0")
    hb = make_host_banks(w)
    sc = oes.schema_make(w.fmt, w.stream_layers, w.E, w.H, w.I)
    L = oes.Layers(sc, 2, 0)
    for layer in range(w.stream_layers):
        for b, t in enumerate(hb.banks):
            L.set_source(b, layer, t)   # one host bank reused under every layer id
    L.prefetch(0)
    logits = synth.router_logits(w.tokens, w.E, 0, w.name).to(dev)
    ids = torch.empty((w.tokens, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.tokens, w.k), dtype=torch.float32, device=dev)
    oes.route_logits(logits, w.k, ids, wts)
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
    out = {"workload": w.name, "tokens": w.tokens, "flops": flops, "ffn_ms": ffn_ms,
           "ffn_TFLOPs": flops / (ffn_ms * 1e9), "ffn_weight_GBps": wbytes / (ffn_ms * 1e6),
           "layer_bytes": wbytes, "layer_copy_ms": copy_ms, "stream_GBps": wbytes / (copy_ms * 1e6),
           "layers": w.stream_layers, "overlapped_ms_per_layer": wall_ms / w.stream_layers}
    log("prefill", {k: (round(v, 3) if isinstance(v, float) else v) for k, v in out.items()})
    L.close()
    return out


def _cpu_baseline(w, hb, x, wg, mr, budget_s, gpu_step=None):
    """The oracle, as it stands, on this host: route + LRU + row copies + FFN for bs=1 steps.

    Its first step also gates the GPU numbers: the routed ids, the slot map, the
    (slot, expert id) misses and the bytes those misses copied into the slot banks in
    the headline step must equal the oracle's, and its FFN output must be within the
    format's tolerance (relative L2 <= 1e-2, 3e-2 for fp4 banks) of the oracle's."""
    import numpy as np

    import synth
    from oracle import copy as ocopy
    from oracle import ffn as offn
    from oracle import route as oroute
    from oracle.lru import SlotTable
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    xb = x.cpu().numpy().view(np.uint16)
    wgb = wg.cpu().numpy().view(np.uint16)
    host = [[hb.banks[b].numpy().reshape(w.E, -1)] for b in range(len(hb.banks))]
    mirror = [np.zeros((w.S, rb), dtype=np.uint8) for rb in hb.row_bytes]
    times = []
    first = None
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 25):
        t0 = time.perf_counter()
        ids, wts, _ = oroute.route(xb, wgb, w.k)
        active = len(set(ids.ravel().tolist()))
        owner, stamp, clock, pre = synth.forced_miss_state(w.S, w.E, 0, ids, int(round(active * mr)))
        t = SlotTable(w.S, w.L, w.E)
        t.set_state(owner, stamp, clock)
        t1 = time.perf_counter()
        r = t.ensure(0, ids)
        ocopy.copy_missing(r.misses, host, mirror, w.E)
        yo = offn.expert_ffn(w.fmt, w.H, w.I, xb, r.slot_ids, wts,
                             lambda s: [host[b][0][int(t.owner[s]) % w.E] for b in range(len(host))])
        t2 = time.perf_counter()
        times.append(((t2 - t1) + (t1 - t0)) * 1000.0)
        if first is None:
            ms_ = sorted((int(sl), int(e)) for sl, e in r.misses)
            first = (ids, r.slot_ids, yo, ms_, [m[[sl for sl, _ in ms_]].copy() for m in mirror])
    ms = float(np.median(times))
    parity = None
    if gpu_step is not None:
        ids_ok = bool(np.array_equal(gpu_step["ids"], first[0]))
        slots_ok = bool(np.array_equal(gpu_step["slot_ids"], first[1]))
        order = np.argsort([sl for sl, _ in gpu_step["misses"]], kind="stable")
        gmiss = [tuple(gpu_step["misses"][i]) for i in order]
        miss_ok = gmiss == first[3]
        bytes_ok = miss_ok and all(np.array_equal(g[order], o) for g, o in zip(gpu_step["rows"], first[4]))
        err = float(offn.rel_l2(gpu_step["y"], first[2]))
        tol = 3e-2 if w.fmt in ("nvfp4", "q4_0") else 1e-2
        parity = {"ids": ids_ok, "slot_ids": slots_ok, "misses": miss_ok, "slot_bytes": bytes_ok,
                  "ffn_rel_l2": err, "ffn_tol": tol,
                  "ok": ids_ok and slots_ok and miss_ok and bytes_ok and err <= tol}
    return {"value": 1000.0 / (w.L * ms), "unit": "tok/s", "cores": int(blas_threads), "kind": "oracle",
            "ms_per_step": ms, "sample": f"{len(times)} bs=1 decode steps of {w.name} at miss_rate {mr} "
                                        f"(route, LRU, row copies, float64 FFN), median",
            "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "parity": parity}


if __name__ == "__main__":
    main()
