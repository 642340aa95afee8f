#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

A step is one moe_forward call (router, top-K gate, dispatch, SwiGLU
experts, combine with the shared expert) over one batch of seeded synthetic
input already resident in HBM.  Prints ONE JSON line.

Default workload: the K2-shaped layer at 16384 tokens (prefill-sized
grouped GEMMs); the 256-token decode-sized batch on the same weights is
measured in the same run and reported under "also".
Per-stage durations come from hipEvents the library records at its stage
boundaries on the launch stream (include/moe.h, MOE_EV_*); the up-projection
stage is a single kernel (the grouped SwiGLU GEMM).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at K2 shape (T=256 decode, T=16384 prefill); % HBM/MFMA peak"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
RIDGE_BF16 = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def work_model(wl, counts):
    """Algorithmic flops and bytes of one forward step and of its up-projection
    kernel.  Bytes: weights of the experts that received tokens read once,
    shared / router / latent weights, x read and out written once (temporaries
    excluded).  Flops: the selected experts' SwiGLU, the shared experts, the
    latent maps; the router counted apart (fp32-class)."""
    es = 2 if wl.act_dtype == "bf16" else 4
    din, F, d, T = wl.d_in, wl.F, wl.d, wl.T
    Fsh = wl.n_shared * wl.F_shared
    A = wl.T * wl.K
    touched = int(sum(1 for c in counts if c > 0))
    w_expert = 3 * din * F * es
    flops_routed = 2.0 * A * 3 * din * F
    flops_shared = 2.0 * T * 3 * d * Fsh
    flops_latent = 2.0 * T * d * wl.d_latent * 2
    flops_router = 2.0 * T * d * wl.E
    bytes_step = (touched * w_expert + 3 * d * Fsh * es + wl.E * d * 4 + wl.E * 4
                  + 2 * d * wl.d_latent * es + 2 * T * d * es)
    up = dict(
        flops=2.0 * A * din * 2 * F + 2.0 * T * d * 2 * Fsh,
        bytes=(touched * 2 * F * din * es + 2 * Fsh * d * es + T * din * es
               + A * F * es + T * Fsh * es),
        unit_flops=2.0 * din * 2 * F, units_flops=A + (T * Fsh / F if F else 0),
        unit_bytes=2 * F * din * es, units_bytes=touched + (Fsh / F if F else 0))
    return dict(touched=touched, flops_bf16=flops_routed + flops_shared + flops_latent,
                flops_router=flops_router, bytes=bytes_step, up=up)


def measure(moe, torch, wl, weights, steps, warmup, seed):
    from moe_inputs import make_router_inputs
    dev = torch.device("cuda:0")
    r_in = make_router_inputs(wl, dev, seed=seed)
    x, W_r, b = r_in["x"], r_in["W_r"], r_in["b"]
    out = torch.empty((wl.T, wl.d), dtype=x.dtype, device=dev)
    ws = moe.Workspace()
    stream = torch.cuda.current_stream()
    kw = dict(n_shared=wl.n_shared, out=out, workspace=ws, stream=stream)
    # one call with the routing returned (untimed): expert histogram
    _, routing = moe.forward(x, W_r, b, weights, wl.K, wl.scale, return_routing=True, **kw)
    counts = routing["counts"].cpu().tolist()
    nev = moe.NUM_STAGE_EVENTS
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    for row in evs:      # create the underlying hipEvents before handing them over
        for e in row:
            e.record(stream)
    for _ in range(warmup):
        moe.forward(x, W_r, b, weights, wl.K, wl.scale, **kw)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        moe.forward(x, W_r, b, weights, wl.K, wl.scale, stage_events=evs[i], **kw)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps
    stages = {}
    for j in range(1, nev):
        name = moe.STAGES[j]
        stages[name] = sum(evs[i][j - 1].elapsed_time(evs[i][j]) for i in range(steps)) / steps
    wm = work_model(wl, counts)
    up_ms = stages["up"]
    up = wm["up"]
    intensity = up["flops"] / up["bytes"]
    if intensity >= RIDGE_BF16:
        ach = up["flops"] / (up_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / PEAK_BF16_TFLOPS, 4), traffic=None,
                    kernel="grouped SwiGLU up-projection (k_gemm, EPI_SWIGLU)",
                    avg_ms=round(up_ms, 4), algorithmic_tflop=round(up["flops"] / 1e12, 4))
    else:
        ach = up["bytes"] / (up_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(ach / PEAK_HBM_GBS, 4), traffic=None,
                    kernel="grouped SwiGLU up-projection (k_gemm, EPI_SWIGLU)",
                    avg_ms=round(up_ms, 4), algorithmic_gb=round(up["bytes"] / 1e9, 3))
    layer_s = ms * 1e-3
    layer = dict(tflops_bf16=round(wm["flops_bf16"] / layer_s / 1e12, 2),
                 mfma_frac=round(wm["flops_bf16"] / layer_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                 gbps=round(wm["bytes"] / layer_s / 1e9, 1),
                 hbm_frac=round(wm["bytes"] / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                 algorithmic_tflop=round(wm["flops_bf16"] / 1e12, 4),
                 algorithmic_gb=round(wm["bytes"] / 1e9, 3),
                 touched_experts=wm["touched"],
                 hist_min_mean_max=[min(counts), round(sum(counts) / len(counts), 2), max(counts)])
    return dict(value=wl.T / layer_s, ms=ms, wall_s=wall, stages={k: round(v, 4) for k, v in stages.items()},
                roofline=roof, layer=layer, inputs=(x, W_r, b))


def cpu_baseline(torch, wl, weights, x, W_r, b, target_s, seed):
    """The oracle as it stands, on a bounded token sample of the same
    workload (router + K routed experts + shared experts per token, fp64,
    OpenMP over tokens)."""
    import numpy as np
    import oracle
    nth = oracle.default_threads()
    xh, Wrh, bh = x.cpu(), W_r.cpu(), b.cpu()
    rng = np.random.default_rng(seed)

    def run(n):
        toks = np.sort(rng.choice(wl.T, size=min(n, wl.T), replace=False))
        xs = xh[toks].contiguous()
        r = oracle.router(xs, Wrh, bh, wl.K, wl.scale, nthreads=nth)   # which experts to copy
        need = set(np.unique(r["idx"]).tolist())
        per = {k: [weights[k][e].cpu() if e in need else None for e in range(wl.E)]
               for k in ("W_gate", "W_up", "W_down")}
        opt = {k: (weights[k].cpu() if weights.get(k) is not None else None)
               for k in ("Ws_gate", "Ws_up", "Ws_down", "W_lat_down", "W_lat_up")}
        lay = oracle.Layer(d=wl.d, E=wl.E, K=wl.K, F=wl.F, scale=wl.scale, W_r=Wrh, b=bh,
                           W_gate=per["W_gate"], W_up=per["W_up"], W_down=per["W_down"],
                           n_shared=wl.n_shared, F_shared=wl.F_shared, Ws_gate=opt["Ws_gate"],
                           Ws_up=opt["Ws_up"], Ws_down=opt["Ws_down"], d_latent=wl.d_latent,
                           W_lat_down=opt["W_lat_down"], W_lat_up=opt["W_lat_up"])
        t = time.perf_counter()
        oracle.forward(lay, xs, nthreads=nth)
        return len(toks), time.perf_counter() - t

    n1, s1 = run(nth)
    n = n1
    s = s1
    if s1 < target_s / 2:
        n2 = int(min(wl.T, max(nth, nth * int(target_s / max(s1, 1e-3)))))
        n2 = min(n2, 32 * nth)
        if n2 > n1:
            n, s = run(n2)
    return dict(value=round(n / s, 3), unit="tokens/s", cores=nth, kind="oracle",
                sample=(f"{n} random tokens of the {wl.T}-token batch, whole layer per token "
                        f"(router over {wl.E} experts, top-{wl.K}, {wl.K} routed + "
                        f"{wl.n_shared} shared SwiGLU experts), fp64, {s:.1f} s"),
                seconds=round(s, 2))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k2_prefill_t16384")
    ap.add_argument("--also", default="k2_decode_t256",
                    help="comma-separated extra workloads on the same weights ('' for none)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="target seconds of oracle time (0 skips the CPU baseline)")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="also run a plain streaming copy (out = in + 0, fp32) of this many GiB "
                         "three times, to scale HBM byte counters (0 = off)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is measured on one GPU's share, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fine_grained_sparse_amd as moe
    from moe_inputs import get_workload, make_expert_weights

    if args.calibrate_copy_gib > 0:
        n = int(args.calibrate_copy_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x (read {n * 4} B, write {n * 4} B)")
        del src, dst
        torch.cuda.empty_cache()
    wl = get_workload(args.workload)
    if wl.router_only:
        sys.exit("choose a whole-layer workload")
    log(f"[bench] generating weights for {wl.name} on the GPU")
    weights = make_expert_weights(wl, "cuda:0", seed=args.seed)
    torch.cuda.synchronize()
    log(f"[bench] timing {wl.name}: warmup {args.warmup}, steps {args.steps}")
    main_r = measure(moe, torch, wl, weights, args.steps, args.warmup, args.seed)
    log(f"[bench] {wl.name}: {main_r['ms']:.3f} ms/step, stages {main_r['stages']}")
    also = {}
    for name in [s for s in args.also.split(",") if s]:
        awl = get_workload(name)
        same = (awl.d, awl.E, awl.F, awl.n_shared, awl.F_shared, awl.d_latent, awl.act_dtype) == \
               (wl.d, wl.E, wl.F, wl.n_shared, wl.F_shared, wl.d_latent, wl.act_dtype)
        if not same:
            log(f"[bench] skipping {name}: different weights")
            continue
        log(f"[bench] timing {name}")
        r = measure(moe, torch, awl, weights, max(args.steps, 20), args.warmup, args.seed)
        log(f"[bench] {name}: {r['ms']:.3f} ms/step, stages {r['stages']}")
        also[name] = dict(value=round(r["value"], 1), unit="tokens/s", ms_per_step=round(r["ms"], 4),
                          roofline=r["roofline"], layer=r["layer"], stages_ms=r["stages"],
                          config=dict(workload=name, T=awl.T))
    cpu = None
    if args.cpu_baseline_seconds > 0:
        log("[bench] CPU baseline (oracle)")
        x, W_r, b = main_r["inputs"]
        cpu = cpu_baseline(torch, wl, weights, x, W_r, b, args.cpu_baseline_seconds, args.seed)
        log(f"[bench] oracle: {cpu['value']} tokens/s on {cpu['cores']} threads")
    line = {
        "metric": METRIC, "value": round(main_r["value"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_r["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.act_dtype,
        "data": "synthetic (seeded N(0,1) x, N(0,1/fan_in) weights, Zipf(1.1) expert skew)",
        "config": dict(workload=wl.name, T=wl.T, d=wl.d, E=wl.E, K=wl.K, F=wl.F,
                       n_shared=wl.n_shared, F_shared=wl.F_shared, d_latent=wl.d_latent,
                       scale=wl.scale, parallelism="single-gpu"),
        "roofline": main_r["roofline"], "cpu_baseline": cpu, "layer": main_r["layer"],
        "stages_ms": main_r["stages"], "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
