"""Benchmark: padding-free MoE layer forward + backward on one MI355X.

Workload (default): the DeepSeek-MoE-16B-like layer -- 4096 tokens, d = 2048,
64 routed SwiGLU experts of hidden 1408, top-6, plus 2 always-on shared experts
of hidden 1408, bf16 with fp32 accumulation, Gaussian synthetic inputs.  One
step is the whole hot path: route, PFT build, dispatch, routed and shared
expert FFN, combine, and the backward of each (combine, experts, dispatch,
router).  Inputs are resident in HBM before the timed region.  --workload
picks another shape; one whose configuration is a forward pass only (the
DeepSeek-V3 shape) times the forward alone and counts its flops alone.

Prints one JSON line: useful TFLOPS (router + routed + shared expert GEMMs on
unpadded rows; backward GEMMs count twice the forward), tokens/s, the roofline
of the dominant kernel (the expert up-projection), and the CPU oracle's
throughput on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd useful TFLOPS + tokens/s on 1 MI355X (DeepSeek-MoE shape)"
# HBM bytes per launch of the up-projection from rocprofv3 FETCH_SIZE / WRITE_SIZE
# runs, per workload, recorded with a hash of the kernel sources they were taken on
COUNTERS = os.path.join(ROOT, "profiles", "up_projection_counters.json")
KERNEL_SOURCES = ["common.hpp", "gemm.hpp", "ffn.hip"]


def kernel_sources_sha1() -> str:
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "padding_free_expert_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """Counter-measured bytes per launch on this workload, or None when the
    counters were taken on another workload or the kernel changed since."""
    try:
        with open(COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha1") != kernel_sources_sha1():
        return None
    return rec.get("workloads", {}).get(workload, {}).get("hbm_bytes_per_launch")


def up_tile(rows: int, E: int, h: int) -> str:
    """The up-projection tile the library picks for a launch (the selection in
    launch_ffn_up, csrc/ffn.hip, repeated here only to name the kernel)."""
    per = rows // max(E, 1)
    large_grid = (rows // 256 + E) * ((h + 127) // 128) >= 512
    if per >= 1024 and large_grid:
        return "gemm_dma_kernel<256,128,32,4,2,2,...,EPI_SWIGLU> (8 waves, 1 block/CU)"
    if h % 256 == 0 and per < 1024:
        return "gemm_dma_kernel<128,256,32,2,4,2,...,EPI_SWIGLU> (8 waves, 1 block/CU)"
    return "gemm_dma_kernel<128,128,32,2,2,2,...,EPI_SWIGLU> (4 waves, 2 blocks/CU)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 30 untimed steps: the first ~25 steps of a process run ~1.5% slower
    # (714-718 against 726-730 TFLOPS timed after 5, 30 or 60 warm-up steps)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="dsmoe16b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the shared experts in order on the main stream")
    ap.add_argument("--merge-shared", action="store_true",
                    help="carry the shared experts as always-routed experts in the routed buffer")
    ap.add_argument("--lean", action="store_true",
                    help="recompute H1/H3 in the backward instead of keeping them from the forward")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens in the oracle's timed sample (0: pick for ~10-30 s)")
    ap.add_argument("--cpu-full", type=int, default=0,
                    help="also time the oracle on the whole workload this many times (median; minutes per run)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale hardware byte counters)")
    ap.add_argument("--timed-only", action="store_true",
                    help="run the warm-up and timed steps only (no cache-flushed steps, per-call breakdown, "
                         "isolated launches, EP/RBD kernels or CPU baseline), so that a profiler's per-kernel "
                         "averages cover exactly the steps whose launches the roofline times")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, repeated; its FETCH_SIZE and
    WRITE_SIZE per dispatch calibrate the counters read on the layer's kernels."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer is not sharded "
              f"across GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads
    import padding_free_expert_amd as xm
    from padding_free_expert_amd.layer import PaddingFreeMoE

    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    assert xm.xmoe_query_device(0), "cuda:0 is not gfx950"
    wl = workloads.get(args.workload)
    assert wl.dtype == "bf16"
    inp = workloads.generate(wl, device="cuda", backward=True)
    weights = {k: inp[k] for k in ("wg", "w1", "w3", "w2", "s1", "s3", "s2", "logit_bias", "select_bias")
               if k in inp}
    # a step is the passes the workload names: forward and backward, or (the
    # DeepSeek-V3 shape) the forward alone
    layer = PaddingFreeMoE(weights, wl.T, wl.k, wl.inv_tau, backward=wl.backward, lean=args.lean,
                           overlap=not args.no_overlap, merge_shared=args.merge_shared)
    x, dy = inp["x"], inp["dy"]
    stream = torch.cuda.current_stream()

    def step(hook=None, probe=None):
        layer.forward(x, hook=hook, probe=probe)
        if wl.backward:
            layer.backward(dy, hook=hook)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    # events right before and after each up-projection launch of the timed
    # steps, on the stream it is launched on (routed: the main stream; shared
    # experts: their side stream)
    up_ev = {"up": [], "shared_up": []}
    up_pool = [torch.cuda.Event(enable_timing=True) for _ in range(4 * args.steps)]

    def probe(name, s):
        e = up_pool.pop()
        e.record(s)
        if name.endswith("_end"):
            up_ev[name[:-4]][-1].append(e)
        else:
            up_ev[name].append([e])

    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(probe=probe)
        marks[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    per_step = [ev0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)]
    up_ms = {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in up_ev.items() if v}

    ms = max(gpu_ms, wall * 1e3 / args.steps)
    flops = wl.useful_flops()
    tflops = flops["total"] / (ms * 1e-3) / 1e12
    tok_s = wl.T / (ms * 1e-3)

    flushed, breakdown = [], {}
    if not args.timed_only:
        # the same steps with the 256 MB Infinity Cache flushed before each one
        # (a 1 GiB scratch write outside the step's events), so no input is
        # served from the last step's cache contents
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        for _ in range(min(args.steps, 10)):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            flushed.append(a.elapsed_time(b))
        del flush

        # per-call breakdown: events between library calls, averaged over a few
        # steps (serially: with the shared experts on their side stream the gaps
        # between main-stream events would not be per-call times)
        names, evs = [], []

        def hook(name):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            names.append(name)
            evs.append(e)

        reps = 5
        overlap = layer.overlap
        layer.overlap = False
        for _ in range(reps):
            names.clear()
            evs.clear()
            start = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            step(hook)
            torch.cuda.synchronize()
            prev = start
            for n, e in zip(names, evs):
                breakdown[n] = breakdown.get(n, 0.0) + prev.elapsed_time(e) / reps
                prev = e
        layer.overlap = overlap

    # roofline of the dominant kernel: the up-projection (W1|W3 + SwiGLU),
    # launched once for the routed experts (rows gathered from x through the
    # PFT's token_ids) and, with shared experts beside them, once for those per
    # step.  Its durations are the timed steps' own launches (events around
    # each launch on its stream, above), so they include whatever the other
    # stream runs at the same time, as a profiler's kernel durations do.
    R, d, h = layer.R, wl.d, wl.h
    launches = [("up", 4.0 * R * d * h,
                 2.0 * (R * d + 2 * layer.Ec * d * h + R * h + (R * 2 * h if layer.h13 is not None else 0)))]
    if layer.side_shared:
        hs = layer.hs
        launches.append(("shared_up", 4.0 * wl.T * d * hs, 2.0 * (wl.T * d + 2 * d * hs + wl.T * hs
                                                                 + (wl.T * 2 * hs if layer.sh_h13 is not None else 0))))
    per, tot_ms, tot_flop, tot_bytes = [], 0.0, 0.0, 0.0
    for name, fl, by in launches:
        t = up_ms[name]
        per.append({"launch": name, "flop": fl, "avg_ms": round(t, 5), "tflops": round(fl / (t * 1e-3) / 1e12, 2)})
        tot_ms += t
        tot_flop += fl
        tot_bytes += by
    if not args.timed_only:
        # the same launches alone, back to back (no other stream running)
        iso = {"up": lambda: xm.xmoe_expert_ffn_up_gather(x, layer.pft.token_ids, layer.W1, layer.W3,
                                                         layer.pft.expert_offsets, layer.act, layer.h13),
               "shared_up": lambda: xm.xmoe_expert_ffn_up(x, weights["s1"].unsqueeze(0), weights["s3"].unsqueeze(0),
                                                          layer.sh_off, layer.sh_act, layer.sh_h13)}
        for p in per:
            launch = iso[p["launch"]]
            for _ in range(3):
                launch()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            p["isolated_avg_ms"] = round(e0.elapsed_time(e1) / 20, 5)
    achieved = tot_flop / (tot_ms * 1e-3) / 1e12
    # the same launches against HBM: each operand read once (the gathered rows,
    # the weights) and each output written once (act, H1|H3)
    hbm_gbps = tot_bytes / (tot_ms * 1e-3) / 1e9
    roofline = {"kernel": "expert up-projection, " + up_tile(R, layer.Ec, h),
                "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic(wl.name),
                "launches_per_step": per, "avg_launch_ms": round(tot_ms / len(launches), 5),
                "timed_steps": args.steps,
                "hbm": {"algorithmic_bytes_per_launch": round(tot_bytes / len(launches)),
                        "achieved_GBps": round(hbm_gbps, 1), "peak_GBps": 8000.0,
                        "frac": round(hbm_gbps / 8000.0, 4)}}

    out = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "h": wl.h, "k": wl.k,
                      "n_shared": wl.n_shared, "h_shared": wl.h_shared,
                      "passes": "fwd+bwd" if wl.backward else "fwd",
                      "h13": ("not kept (forward only)" if not wl.backward else
                              "recomputed" if args.lean else "saved"),
                      "shared_experts": ("merged as always-routed experts" if layer.merged else
                                         "side stream" if layer.side_shared and layer.overlap else
                                         "in order" if layer.shared else "none")},
           "tokens_per_s": round(tok_s, 1), "gpu_ms_per_step": round(gpu_ms, 4),
           "step_ms": pctl(per_step),
           "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
           "useful_gflop_per_step": round(flops["total"] / 1e9, 2),
           "saved_activation_mb": round(layer.saved_bytes() / 1e6, 1),
           "roofline": roofline}
    if args.timed_only:
        print(json.dumps(out), flush=True)
        return
    out["step_ms_cache_flushed"] = pctl(flushed)
    out["value_cache_flushed"] = round(flops["total"] / (out["step_ms_cache_flushed"]["median"] * 1e-3) / 1e12, 2)
    out["breakdown_ms_serial"] = {k: round(v, 4) for k, v in breakdown.items()}
    roofline["per_product"] = per_product(xm, wl, layer, weights, x, dy, stream)
    # the products alone leave the layer's buffers with partial results (the
    # dispatch backward without the shared experts' input gradient): one more
    # whole step restores them before anything below reads the outputs
    step()
    torch.cuda.synchronize()
    out["ep_rbd"] = ep_rbd(xm, wl, layer, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline(wl, inp, args.cpu_sample_tokens, layer, args.cpu_full)
    print(json.dumps(out), flush=True)


def per_product(xm, wl, layer, weights, x, dy, stream, reps=20):
    """Every product of the step alone: 3 untimed calls, then `reps` calls back
    to back between two events, on the layer's own buffers (after the timed
    steps, so they hold one step's values; some calls overwrite outputs with
    partial results, so the caller reruns a whole step afterwards).  Matrix-core products report
    TFLOP/s against the bf16 peak; the row kernels, the router and its
    backward report algorithmic GB/s against HBM (each input read once, each
    output written once), the PFT build microseconds."""
    import torch

    T, d, E, h, k = wl.T, wl.d, wl.E, wl.h, wl.k
    R, Ec, off, pft = layer.R, layer.Ec, layer.pft.expert_offsets, layer.pft
    kc = layer.kc
    rows = {}

    def run(name, fn, flop=None, nbytes=None):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        r = {"ms": round(ms, 5)}
        if flop is not None:
            tf = flop / (ms * 1e-3) / 1e12
            r.update(gflop=round(flop / 1e9, 2), tflops=round(tf, 1), frac=round(tf / PEAK_BF16_TFLOPS, 4))
        if nbytes is not None:
            gb = nbytes / (ms * 1e-3) / 1e9
            r.update(mbytes=round(nbytes / 1e6, 1), GBps=round(gb, 1), frac_hbm=round(gb / PEAK_HBM_GBS, 4))
        rows[name] = r

    w = layer.w
    s = 2  # bytes per bf16 element
    run("route", lambda: xm.xmoe_route(x, w["wg"], k, layer.topk_ids, layer.topk_w, layer.logits, layer.inv_tau,
                                       w.get("logit_bias"), w.get("select_bias"), workspace=layer.route_ws),
        flop=2.0 * T * d * E, nbytes=T * d * s + d * E * s + 4.0 * T * E + 8.0 * T * k)
    if layer.merged:
        run("build_pft", lambda: xm.xmoe_build_pft_shared(layer.topk_ids, layer.topk_w, E, layer.ns, pft,
                                                          layer.pft_ws))
    else:
        run("build_pft", lambda: xm.xmoe_build_pft(layer.topk_ids, layer.topk_w, E, pft, layer.pft_ws))
    h13 = layer.h13
    run("up", lambda: xm.xmoe_expert_ffn_up_gather(x, pft.token_ids, layer.W1, layer.W3, off, layer.act, h13),
        flop=4.0 * R * d * h)
    run("down", lambda: xm.xmoe_expert_ffn_down(layer.act, layer.W2, off, layer.ye), flop=2.0 * R * d * h)
    y_add = layer.sh_y if layer.side_shared else None
    run("combine", lambda: xm.xmoe_combine(layer.ye, pft, T, layer.y, y_add=y_add),
        nbytes=R * d * s + T * d * s * (2 if y_add is not None else 1) + 8.0 * R)
    if layer.side_shared:
        hs, so = layer.hs, layer.sh_off
        s1, s3, s2 = layer._shared_w()
        run("shared_up", lambda: xm.xmoe_expert_ffn_up(x, s1, s3, so, layer.sh_act, layer.sh_h13),
            flop=4.0 * T * d * hs)
        run("shared_down", lambda: xm.xmoe_expert_ffn_down(layer.sh_act, s2, so, layer.sh_y), flop=2.0 * T * d * hs)
    if wl.backward:
        run("combine_bwd", lambda: xm.xmoe_combine_bwd(dy, layer.ye, pft, layer.dye, layer.dtopk_w_all),
            nbytes=T * d * s + 2.0 * R * d * s + 12.0 * R)
        run("dact", lambda: xm.xmoe_expert_ffn_bwd_dact_gather(dy, pft.token_ids, pft.combine_weights, layer.W2, h13,
                                                             off, layer.dh13),
            flop=2.0 * R * d * h)
        run("dx", lambda: xm.xmoe_expert_ffn_bwd_dx(layer.dh13, layer.W1, layer.W3, off, layer.dxs),
            flop=4.0 * R * d * h)
        run("dw13", lambda: xm.xmoe_expert_ffn_bwd_dw13_gather(x, pft.token_ids, layer.dh13, off, layer.dW1,
                                                               layer.dW3), flop=4.0 * R * d * h)
        run("dw2", lambda: xm.xmoe_expert_ffn_bwd_dw2(layer.act, layer.dye, off, layer.dW2), flop=2.0 * R * d * h)
        if layer.side_shared:
            run("shared_dact", lambda: xm.xmoe_expert_ffn_bwd_dact(dy, s2, layer.sh_h13, so, layer.sh_dh13),
                flop=2.0 * T * d * hs)
            run("shared_dx", lambda: xm.xmoe_expert_ffn_bwd_dx(layer.sh_dh13, s1, s3, so, layer.sh_dx),
                flop=4.0 * T * d * hs)
            run("shared_dw13", lambda: xm.xmoe_expert_ffn_bwd_dw13(x, layer.sh_dh13, so, layer._ds1, layer._ds3),
                flop=4.0 * T * d * hs)
            run("shared_dw2", lambda: xm.xmoe_expert_ffn_bwd_dw2(layer.sh_act, dy, so, layer._ds2),
                flop=2.0 * T * d * hs)
        rdx = layer.rdx
        run("route_bwd", lambda: xm.xmoe_route_bwd(x, w["wg"], layer.logits, layer.topk_ids, layer.dtopk_w, rdx,
                                                   layer.dwg, layer.rbwd_ws, layer.inv_tau, accumulate=False),
            flop=4.0 * T * d * E, nbytes=4.0 * T * E + 8.0 * R + 2.0 * T * d * s + 4.0 * d * E)
        run("dispatch_bwd", lambda: xm.xmoe_dispatch_bwd(layer.dxs, pft, T, layer.dx, dx_add=rdx),
            nbytes=R * d * s + 2.0 * T * d * s + 4.0 * R)
    return rows


def pctl(v):
    """median, p10 and p90 of a list of step times (ms)."""
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def ep_rbd(xm, wl, layer, stream, nodes=8, ranks=8, n_rep=20):
    """Time the expert-parallel plans and the pilot-token build at this shape:
    pilots of the layer's own routing over `nodes` nodes; the send plan of its
    buffer over `ranks` ranks; the receive plan and regroup of rank 0 fed by
    `ranks` sources with independent routings of the same shape."""
    import torch
    import workloads

    T, E, k, d = wl.T, wl.E, wl.k, wl.d
    if E % nodes or E % ranks:
        return None
    i32 = dict(dtype=torch.int32, device="cuda")

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_rep):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_rep * 1e3  # us

    ids = layer.topk_ids
    pl = [torch.empty((T * k,), **i32) for _ in range(3)]
    nc, no = torch.empty((nodes,), **i32), torch.empty((nodes + 1,), **i32)
    pws = torch.empty(max(xm.xmoe_build_pilots_workspace_size(T, E, k, E // nodes), 16), dtype=torch.uint8,
                      device="cuda")
    t_pil = timed(lambda: xm.xmoe_build_pilots(ids, E, E // nodes, pl[0], pl[1], nc, no, pl[2], pws))
    n_pilots = int(no[-1].item())

    sc, sd = torch.empty((ranks,), **i32), torch.empty((ranks + 1,), **i32)
    # the routed experts' part of the buffer (shared experts stay on every rank)
    routed_off = layer.pft.expert_offsets[:E + 1]
    t_send = timed(lambda: xm.xmoe_ep_send_plan(routed_off, ranks, sc, sd))

    el = E // ranks
    C = torch.stack([torch.bincount(workloads.random_topk(T, E, k, seed=100 + s)[0].reshape(-1).long(),
                                    minlength=E)[:el] for s in range(ranks)]).to(torch.int32)
    n = int(C.sum())
    Cd = C.cuda()
    lo, rd = torch.empty((el + 1,), **i32), torch.empty((ranks + 1,), **i32)
    l2r, r2l = torch.empty((n,), **i32), torch.empty((n,), **i32)
    rws = torch.empty(max(xm.xmoe_ep_recv_plan_workspace_size(ranks, el), 16), dtype=torch.uint8, device="cuda")
    t_recv = timed(lambda: xm.xmoe_ep_recv_plan(Cd, n, lo, rd, l2r, r2l, rws))
    rows = torch.randn(n, d, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(rows)
    t_reg = timed(lambda: xm.xmoe_scatter_rows(rows, r2l, dst))
    # the same regroup with the 256 MB Infinity Cache flushed before each call
    # (its ~100 MB working set otherwise stays cache-resident between calls)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    t_fl = 0.0
    for _ in range(n_rep):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        xm.xmoe_scatter_rows(rows, r2l, dst)
        e1.record(stream)
        torch.cuda.synchronize()
        t_fl += e0.elapsed_time(e1) * 1e3 / n_rep
    del flush
    moved = 2.0 * n * d * 2 + 4.0 * n  # rows read and written once, plus the index
    return {"pilots": {"nodes": nodes, "experts_per_node": E // nodes, "us": round(t_pil, 2),
                       "pilots": n_pilots, "slots": T * k, "pilot_fraction": round(n_pilots / (T * k), 4)},
            "send_plan": {"ranks": ranks, "us": round(t_send, 2)},
            "recv_plan": {"ranks": ranks, "rows": n, "us": round(t_recv, 2)},
            "regroup": {"rows": n, "d": d, "us_cache_resident": round(t_reg, 2),
                        "GB_per_s_cache_resident": round(moved / (t_reg * 1e-6) / 1e9, 1),
                        "us_cache_flushed": round(t_fl, 2),
                        "GB_per_s_cache_flushed": round(moved / (t_fl * 1e-6) / 1e9, 1)}}


def cpu_info():
    """CPU model, sockets and the threads this process may use (lscpu, else
    /proc/cpuinfo)."""
    info = {"model": None, "sockets": None, "threads_available": len(os.sched_getaffinity(0))}
    try:
        import subprocess
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in txt.splitlines():
            key, _, val = line.partition(":")
            if key.strip() == "Model name":
                info["model"] = val.strip()
            elif key.strip() == "Socket(s)":
                info["sockets"] = int(val.strip()) if val.strip().isdigit() else val.strip()
    except (OSError, ValueError):
        pass
    if info["model"] is None:
        try:
            with open("/proc/cpuinfo") as fh:
                for line in fh:
                    if line.startswith("model name"):
                        info["model"] = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    return info


def oracle_tiny_single_thread(reps=3):
    """The oracle's forward of the tiny fp32 workload (256 tokens, d 128, 8
    experts of 64, top-2) on one thread, median of `reps` runs."""
    import numpy as np

    import oracle as orc
    import workloads

    wl = workloads.get("tiny_f32")
    inp = workloads.generate(wl, backward=False)
    o = {k: v.numpy() for k, v in inp.items() if v is not None}
    prev = orc.get_threads()
    orc.set_threads(1)
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        orc.layer_forward(o, wl.k, 0, wl.inv_tau)
        ts.append(time.perf_counter() - t0)
    orc.set_threads(prev)
    t = float(np.median(ts))
    return {"workload": "tiny_f32 forward", "threads": 1, "seconds_median": round(t, 5), "runs": reps,
            "gflops": round(wl.useful_flops()["fwd"] / t / 1e9, 3), "tokens_per_s": round(wl.T / t, 1)}


def cpu_baseline(wl, inp, sample_tokens, layer, full_runs=0):
    """The CPU oracle, as it stands, on the first `sample_tokens` tokens of the
    same inputs: full forward and backward (routing, experts, shared experts,
    combine, all gradients) for those tokens; throughput scaled per token.
    Its y and dx of those tokens also check the GPU run's own outputs (both are
    per token): normwise relative error over the tokens whose top-k agrees with
    the oracle's (a near-tie may order two experts differently)."""
    import numpy as np
    import torch

    import oracle as orc

    cores = len(os.sched_getaffinity(0))
    orc.set_threads(cores)

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    n = sample_tokens or 512
    o = {k: bits(v) for k, v in inp.items() if v is not None and k not in ("logit_bias", "select_bias")}
    for k in ("logit_bias", "select_bias"):
        if inp.get(k) is not None:
            o[k] = inp[k].cpu().numpy()
    o["x"] = o["x"][:n]
    o["dy"] = o["dy"][:n]
    t0 = time.perf_counter()
    fwd = orc.layer_forward(o, wl.k, 1, wl.inv_tau, n_shared=wl.n_shared)
    bwd = orc.layer_backward(o, fwd, o["dy"], wl.inv_tau, n_shared=wl.n_shared) if wl.backward else None
    dt = time.perf_counter() - t0
    sub = wl.__class__(**{**wl.__dict__, "T": n})
    fl = sub.useful_flops()["total"]
    what = "full forward+backward incl. all weight gradients" if wl.backward else "full forward"
    base = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOPS", "cores": orc.get_threads(), "kind": "oracle",
            "sample": f"{n} of {wl.T} tokens, {what}",
            "seconds": round(dt, 2), "tokens_per_s": round(n / dt, 2), "cpu": cpu_info(),
            "single_thread_tiny": oracle_tiny_single_thread()}
    if full_runs > 0:
        # the whole workload, as many runs as asked (median).  Every token's
        # forward and backward is independent of the others', so a run is
        # timed over token chunks of about a minute each (sized from the
        # sample's rate), the same work in total; the weight gradients of the
        # chunks are not summed (only the time is kept).
        import numpy as np
        X, DY = bits(inp["x"]), bits(inp["dy"])
        per_tok = dt / n
        chunk = wl.T
        while chunk > 256 and chunk * per_tok > 60.0:
            chunk //= 2
        nch = (wl.T + chunk - 1) // chunk
        ts = []
        for _ in range(full_runs):
            tot = 0.0
            for c in range(nch):
                part = {k: v for k, v in o.items()}
                part["x"] = X[c * chunk:(c + 1) * chunk]
                part["dy"] = DY[c * chunk:(c + 1) * chunk]
                t1 = time.perf_counter()
                f2 = orc.layer_forward(part, wl.k, 1, wl.inv_tau, n_shared=wl.n_shared)
                if wl.backward:
                    orc.layer_backward(part, f2, part["dy"], wl.inv_tau, n_shared=wl.n_shared)
                tot += time.perf_counter() - t1
                if nch > 1:
                    print(f"oracle full run {len(ts) + 1}/{full_runs}, chunk {c + 1}/{nch}: {tot:.1f} s",
                          file=sys.stderr, flush=True)
            ts.append(tot)
            print(f"oracle full run {len(ts)}/{full_runs}: {ts[-1]:.1f} s", file=sys.stderr, flush=True)
        tm = float(np.median(ts))
        base["full_workload"] = {"tokens": wl.T, "runs": full_runs, "chunks": nch, "seconds_median": round(tm, 2),
                                 "tflops": round(wl.useful_flops()["total"] / tm / 1e12, 6),
                                 "tokens_per_s": round(wl.T / tm, 2)}
    ok = (layer.topk_ids[:n].cpu().numpy() == fwd["route"]["topk_ids"]).all(axis=1)

    def rel(g, r):
        g = g[:n].detach().cpu().to(torch.float64).numpy()[ok]
        return float(np.linalg.norm(g - r[ok]) / max(np.linalg.norm(r[ok]), 1e-300))
    ry = rel(layer.y, fwd["y"])
    rdx = rel(layer.dx, bwd["dx"]) if wl.backward else None
    tol = 2e-2
    parity = {"tokens": n, "tokens_compared": int(ok.sum()), "y_rel_err": ry, "dx_rel_err": rdx, "rtol": tol,
              "pass": bool(ry <= tol and (rdx is None or rdx <= tol)), "against": "oracle (fp64) on the same inputs"}
    return base, parity


if __name__ == "__main__":
    main()
