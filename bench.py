"""Benchmark of the fused FP8 MoE expert layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|mid|prefill|wide|tiny]
                (any of decode, mid, prefill, tiny with the suffix _mxfp4: MXFP4 weights)

A step is one forward of the whole layer (dispatch, the persistent expert
kernel, combine) over one batch of seeded synthetic inputs already resident in
HBM.  Prints one JSON line.  The default workload is the 128-token decode
batch (hidden 7168, intermediate 2048, 32 local experts, top-8, uniform
routing), which is weight-stream bound: ``value`` is the achieved
weight-stream rate (bytes of the active experts' FP8 weights and scales per
step / step time); the prefill workload reports FP8 TFLOP/s instead.  With
the decode workload the line also carries ``prefill``: the same measurement
of the 8192-token prefill batch (Zipf(1.2) routing), the compute-bound half
of the metric, in the same process with the same step counts; it is measured
first, so that the decode steps run on a GPU already under load (a GPU that
has been idle needs about 15 ms of work to reach its steady clock).

W untimed warm-up steps, then the K timed steps, twice.  The first pass is
plain: its wall time, bracketed by device synchronisations, gives
``ms_per_step`` and ``value``.  The second pass records HIP events on the
layer's stream around each kernel group of every step; these per-launch
durations give ``kernel_ms`` and the ``roofline`` of the dominant kernel (the
persistent expert kernel).  The events add a few microseconds per step,
which is why they stay out of the first pass.  ``roofline.achieved`` is the
algorithmic work per launch over the expert kernel's mean event time: the
compulsory bytes (the active experts' weights and scales, x and its scales,
the top-k ids and weights, y) for the HBM-bound workloads, 6*H*I FLOPs per
route for prefill.  The intermediates the method writes and reads back
(re-quantised activations, BF16 partials) are reported beside it, not
counted.  ``cpu_baseline`` times the float64 CPU oracle on this host on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix peak
METRIC = "MoE layer FP8 TFLOPS & weight-stream HBM GB/s (decode/prefill), % roofline"


def work_of(inp):
    """Algorithmic work of one step (routing-dependent, exact for these inputs)."""
    x, idx = inp["x"], inp["topk_idx"]
    T, H = x.shape
    mx = "w1_fp4" in inp
    E, N, _ = inp["w1_fp4" if mx else "w1"].shape
    I = N // 2
    k = idx.shape[1]
    act = (idx >= 0) & (idx < E)
    R = int(act.sum())
    active_experts = int(len(np.unique(idx[act])))
    flops = 6.0 * H * I * R
    if mx:   # E2M1 pairs + one UE8M0 byte per 32 K of every row
        w_bytes = active_experts * (3.0 * H * I / 2 + 3.0 * H * I / 32)
    else:
        w_bytes = active_experts * (3.0 * H * I + 4.0 * (2 * I // 128) * (H // 128)
                                    + 4.0 * (H // 128) * (I // 128))
    # compulsory bytes: the active experts' weights and scales, x and its
    # scales, the top-k ids and weights, y
    io_bytes = T * H + 4.0 * T * (H // 128) + 8.0 * T * k + 2.0 * T * H
    # intermediates the method itself writes and reads back (not part of the
    # roofline, reported beside it): re-quantised activations and their
    # scales, BF16 partials
    inter_bytes = R * (2.0 * (I + 4.0 * (I // 64)) + 2.0 * 2.0 * H)
    return dict(T=T, H=H, I=I, E=E, k=k, R=R, active_experts=active_experts, flops=flops, mx=mx,
                weight_bytes=w_bytes, compulsory_bytes=w_bytes + io_bytes,
                intermediate_bytes=inter_bytes)


def _blas_threads():
    """Threads of the BLAS the oracle's matrix products run on."""
    try:
        from threadpoolctl import threadpool_info
        n = [d["num_threads"] for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(name, inp, work):
    """Time the oracle on a bounded sample of the workload on this host."""
    from oracle import moe
    cores = _blas_threads()
    T = inp["x"].shape[0]
    if T <= 128:
        # whole forwards, best of 3 (about 10 s of CPU work at the decode size)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            moe.forward(inp)
            times.append(time.perf_counter() - t0)
        dt = min(times)
        sample = f"full {name} workload ({T} tokens), best of 3 forwards"
        frac = 1.0
    else:
        n = 64
        toks = list(range(n))
        t0 = time.perf_counter()
        moe.forward_tokens(inp, toks)
        dt = time.perf_counter() - t0
        sample = f"first {n} of {T} tokens of the {name} workload, scaled by routes"
        frac = float(((inp["topk_idx"][:n] >= 0) & (inp["topk_idx"][:n] < work["E"])).sum()) / work["R"]
    if name.startswith("prefill"):
        value, unit = work["flops"] * frac / dt / 1e12, "TFLOP/s"
    else:
        value, unit = work["weight_bytes"] / (dt / frac) / 1e9, "GB/s"
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "sample": sample,
            "seconds": dt, "blas": "numpy float64"}


# With L1 on the exact F16 matrix path (two thirds of the FLOPs at the F16
# rate, 2.5 PFLOP/s) and L2 on FP8 (one third at 5.0 PFLOP/s), the layer's own
# ceiling at full MFMA use is 1 / (2/3 / 2.5 + 1/3 / 5.0) = 3.0 PFLOP/s.
EXACT_PATH_PEAK_TFLOPS = 1.0 / ((2.0 / 3.0) / 2500.0 + (1.0 / 3.0) / 5000.0)


def prepare(name, args, torch, B, S, RS):
    """Inputs of one workload generated on the host and resident on the GPU,
    a layer handle sized for it, and the host-side look-ups of its result:
    everything that is not a step happens before the first step."""
    inp = S.make_inputs(name)
    work = work_of(inp)
    wkeys = ("w1_fp4", "w1_e8", "w2_fp4", "w2_e8") if work["mx"] else ("w1", "w1_sf", "w2", "w2_sf")
    dev = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to("cuda:0")
           for k in ("x", "x_sf", "topk_idx", "topk_weights") + wkeys}
    T, H = inp["x"].shape
    y = torch.empty((T, H), dtype=torch.int16, device="cuda:0")
    layer = B.MegaMoE(work["E"], H, work["I"], work["k"], T, block_m=args.block_m,
                      block_n=args.block_n, l2_n_major=args.l2_n_major,
                      split_l2_cus=args.split_l2_cus, split_l2_xcds=args.split_l2_xcds)
    plan = B.mega_moe_plan(layer.cfg, T)
    fwd = layer.forward_mxfp4 if work["mx"] else layer.forward

    def step():
        fwd(dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_weights"], dev[wkeys[0]],
            dev[wkeys[1]], dev[wkeys[2]], dev[wkeys[3]], y)

    # calibrated HBM bytes per launch from the committed counter summary of
    # this workload; None when the library sources changed since it was taken
    # (hashing the sources takes long enough that, done between two timed
    # workloads, it let the GPU's clock drop)
    traffic = RS.read_traffic(os.path.join(ROOT, "profiles", f"moe_expert_ffn_{name}_hbm_traffic.txt"), name)
    return dict(name=name, inp=inp, work=work, dev=dev, y=y, layer=layer, plan=plan, step=step,
                traffic=traffic)


def measure(ctx, args, torch, B):
    """Times `args.steps` forwards of a prepared workload after `args.warmup`
    untimed ones.  Only the raw times are kept here (in ctx); `result` builds
    the result after every workload is timed, since its first call costs tens
    of milliseconds of one-time host work (numpy's first median and the
    like), and a GPU idle that long between two workloads starts the second
    on a lower clock (measured: a 35 ms gap put the decode expert kernel at
    263-267 us against 243-245 without it)."""
    name, layer, step = ctx["name"], ctx["layer"], ctx["step"]
    for _ in range(args.warmup):
        step()
    status = layer.status()
    if status:
        raise SystemExit(f"{name}: device error bits {status:#x}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the same steps again, with HIP events around each kernel group
    B.mega_moe_profile_begin(layer.handle, args.steps)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    prof = B.mega_moe_profile_end(layer.handle, args.steps)
    status = layer.status()
    if status:
        raise SystemExit(f"{name}: device error bits {status:#x}")
    ctx["times"] = (t0, t1, t2, t3, prof)


def result(ctx, args):
    """The result dict of a measured workload: (inputs, work, result)."""
    name, inp, work, plan = ctx["name"], ctx["inp"], ctx["work"], ctx["plan"]
    t0, t1, t2, t3, prof = ctx["times"]
    T, H = inp["x"].shape

    ms = (t1 - t0) * 1e3 / args.steps
    s = ms / 1e3
    k_ms = np.array(prof)                      # [steps, 3] dispatch / expert / combine
    expert_ms = float(k_ms[:, 1].mean())
    tflops = work["flops"] / s / 1e12
    wgbs = work["weight_bytes"] / s / 1e9
    t_roof = max(work["compulsory_bytes"] / (HBM_PEAK_GBS * 1e9), work["flops"] / (FP8_PEAK_TFLOPS * 1e12))
    if name.startswith("prefill"):
        value, unit = tflops, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": work["flops"] / (expert_ms / 1e3) / 1e12,
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        value, unit = wgbs, "GB/s"
        roof = {"bound": "hbm", "achieved": work["compulsory_bytes"] / (expert_ms / 1e3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = ctx["traffic"]
    roof["algorithmic_bytes"] = work["compulsory_bytes"]
    roof["algorithmic_flops"] = work["flops"]
    roof["intermediate_bytes"] = work["intermediate_bytes"]
    if roof["bound"] == "mfma":
        roof["exact_path_peak"] = EXACT_PATH_PEAK_TFLOPS
        roof["frac_of_exact_path_peak"] = roof["achieved"] / EXACT_PATH_PEAK_TFLOPS
    roof["kernel"] = (f"moe_expert_ffn<{plan.block_m}x128, mxfp4>" if work["mx"]
                      else f"moe_expert_ffn<{plan.block_m}x{plan.block_n}>")
    roof["kernel_ms"] = expert_ms
    res = {
        "value": value, "unit": unit, "ms_per_step": ms,
        "config": {"workload": name, "tokens": T, "hidden": H, "intermediate": work["I"],
                   "experts": work["E"], "topk": work["k"], "routing": inp["workload"].routing,
                   "block_m": plan.block_m, "block_n": 128 if work["mx"] else plan.block_n,
                   "weights": "mxfp4" if work["mx"] else "fp8",
                   "split_l2_cus": args.split_l2_cus, "split_l2_xcds": args.split_l2_xcds,
                   "l2_n_major": plan.l2_n_major},
        "tflops": tflops, "weight_stream_gbs": wgbs,
        "pct_roofline": 100.0 * t_roof / s,
        "kernel_ms": {"dispatch": float(k_ms[:, 0].mean()), "expert": expert_ms,
                      "combine": float(k_ms[:, 2].mean())},
        # per-step event times of the same kernels: median and minimum
        "kernel_ms_median": {n: float(np.median(k_ms[:, i]))
                             for i, n in enumerate(("dispatch", "expert", "combine"))},
        "kernel_ms_min": {n: float(k_ms[:, i].min())
                          for i, n in enumerate(("dispatch", "expert", "combine"))},
        "ms_per_step_with_events": (t3 - t2) * 1e3 / args.steps,
        "roofline": roof,
    }
    return inp, work, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps of each workload")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--block-n", type=int, default=0)
    ap.add_argument("--l2-n-major", type=int, default=-1)
    ap.add_argument("--split-l2-cus", type=int, default=0,
                    help="run L1 and L2 tiles as two concurrent kernels, the L2 one with this "
                         "many CUs' worth of workgroups per XCD (0: one fused kernel)")
    ap.add_argument("--split-l2-xcds", type=int, default=0,
                    help="L1 and L2 tiles on disjoint XCD sets: the last n XCDs take the L2 tiles")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the decode workload, skip the prefill measurement that the "
                         "line otherwise carries under \"prefill\"")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the layer is one GPU's share of expert "
              f"parallelism; no multi-GPU path is built); got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_mixture_experts_amd import binding as B
    from fp8_mixture_experts_amd import synthetic as S
    from fp8_mixture_experts_amd import rocprof_summary as RS

    name = args.workload
    pre = None
    with_prefill = name == "decode" and not args.no_prefill
    # Both workloads' inputs are generated and uploaded before any timing:
    # building the decode inputs on the host takes seconds, and a GPU left
    # idle that long starts the next steps on a lower clock (measured on
    # MI355X: decode expert kernels of 280-300 us for the first 20 steps after
    # a 2 s pause, 242 us steady, 245 us from the first step when they follow
    # the prefill steps directly).
    # Nothing is freed until every workload is timed either: after the
    # prefill buffers were freed the next 60 decode steps ran at 260-311 us
    # per expert kernel (245-249 us with them kept); and between the two
    # workloads nothing runs on the host but the timing itself.
    pctx = prepare("prefill", args, torch, B, S, RS) if with_prefill else None
    ctx = prepare(name, args, torch, B, S, RS)
    if with_prefill:
        # the compute-bound half of the metric: the 8192-token prefill batch,
        # the same number of warm-up and timed steps.  It runs first, so the
        # decode steps are then timed on a GPU under load, as in a running
        # model, rather than on one ramping up from idle.
        measure(pctx, args, torch, B)
    measure(ctx, args, torch, B)
    if with_prefill:
        _, _, pre = result(pctx, args)
    inp, work, res = result(ctx, args)
    for c in (pctx, ctx):
        if c is not None:
            c["layer"].close()
            c.clear()
    out = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 x mxfp4" if work["mx"] else "fp8_e4m3", "data": "synthetic",
    }
    out.update({k: v for k, v in res.items() if k not in ("value", "unit", "ms_per_step")})
    if pre is not None:
        out["prefill"] = pre
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        out["copy_probe_bytes"] = args.copy_probe_mib << 20
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, inp, work)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
