"""Launch the decode expert FFN alone, cold, for profiling with rocprofv3.

    python -m offloaded_expert_slot_amd.profile_ffn --workload bf16_h2048 --bs 1 [--launches 64] [--path auto]

Sets up the workload's cache with its layer-0 host banks registered under layers
0..R-1, copies the experts routed for `bs` seeded tokens into R disjoint slot sets
(one per layer, every slot first owned by a layer no step uses), then runs 4
untimed FFN launches followed by `launches` timed ones that cycle over the R sets,
so that no launch finds the previous launches' rows in the memory-side cache
(the bench's cold FFN measurement).  Prints the mean time per launch and the
distinct experts' bytes per launch.  Every FFN kernel dispatched after the first
4 launches belongs to the timed loop, which makes counter windows simple.

--calibrate first reads 1 GiB with the HBM read probe and fills 1 GiB with torch:
kernels of known traffic in the same process, which give the scale factors of the
FETCH_SIZE and WRITE_SIZE counters.
"""
import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="bf16_h2048")
    ap.add_argument("--bs", type=int, default=1)
    ap.add_argument("--launches", type=int, default=64)
    ap.add_argument("--path", choices=("auto", "per_pair", "grouped"), default="auto")
    ap.add_argument("--calibrate", action="store_true", help="a 1 GiB read and a 1 GiB fill first")
    args = ap.parse_args()

    import torch

    import offloaded_expert_slot_amd as oes
    import synth
    from synth.workloads import WORKLOADS, make_host_banks

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.calibrate:
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        sink = torch.zeros(4, dtype=torch.float32, device=dev)
        oes.probe_hbm_read(buf, buf.numel(), sink)
        torch.cuda.synchronize()
        del buf, sink
        torch.cuda.empty_cache()
    hb = make_host_banks(w)
    sc = oes.schema_make(w.fmt, w.L, w.E, w.H, w.I)
    cache = oes.Cache(sc, w.S, 0)
    cache.set_option(oes.OPT_FFN_PATH, {"auto": oes.FFN_AUTO, "per_pair": oes.FFN_PER_PAIR,
                                        "grouped": oes.FFN_GROUPED}[args.path])
    x = synth.activations(args.bs, w.H, 0, w.name, step=101).to(dev)
    wg = synth.router_weight(w.H, w.E, 0, w.name).to(dev)
    ids = torch.empty((args.bs, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((args.bs, w.k), dtype=torch.float32, device=dev)
    oes.route(x, wg, w.k, ids, wts, torch.empty(oes.route_workspace_bytes(args.bs, w.H, w.E), dtype=torch.uint8,
                                                  device=dev))
    torch.cuda.synchronize()
    u = len(set(ids.cpu().numpy().ravel().tolist()))
    R = max(1, min(16, w.S // u, w.L))
    for layer in range(R):
        for b, t in enumerate(hb.banks):
            cache.set_source(b, layer, t)
    owner, stamp, clock = synth.foreign_state(w.S, w.E)
    cache.set_state(owner + (w.L - 1) * w.E, stamp, clock)
    maps = []
    for layer in range(R):
        sl = torch.empty_like(ids)
        cache.ensure_experts(layer, ids, sl)
        cache.copy_missing()
        maps.append(sl)
    y = torch.empty((args.bs, w.H), dtype=torch.int16, device=dev)
    ws = torch.empty(cache.ffn_workspace_bytes(args.bs, w.k), dtype=torch.uint8, device=dev)
    for i in range(4):
        cache.expert_ffn(x, maps[i % R], wts, y, ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.launches):
        cache.expert_ffn(x, maps[i % R], wts, y, ws)
    b.record()
    torch.cuda.synchronize()
    cache.check()
    ms = a.elapsed_time(b) / args.launches
    nbytes = u * sc.bytes_per_expert
    print(f"{w.name} bs={args.bs} path={args.path} distinct experts {u} bytes/launch {nbytes} "
          f"mean {ms * 1e3:.2f} us = {nbytes / (ms * 1e6):.1f} GB/s over {R} disjoint sets", flush=True)
    cache.close()


if __name__ == "__main__":
    main()
