#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

A step is one moe_forward call (router, top-K gate, dispatch, SwiGLU
experts, combine with the shared expert) over one batch of seeded synthetic
input already resident in HBM.  Prints ONE JSON line.

Default workload: the K2-shaped layer at 16384 tokens (prefill-sized
grouped GEMMs).  Measured in the same run and reported under "also": the
256-token decode batch on the same weights, the router alone at 4096
tokens, and the K3-shaped latent layer.
Per-stage durations come from hipEvents the library records at its stage
boundaries on the launch stream (include/moe.h, MOE_EV_*); the up-projection
stage is a single kernel (the grouped SwiGLU GEMM), the one the "roofline"
object describes.  Its "traffic" is read from profiles/up_gemm_hbm_traffic.md when that
table holds a row for the workload taken with the current kernel sources
(otherwise null); `--summarize-counters` writes such rows from two
rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) of this script.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
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
TRAFFIC_MD = os.path.join(ROOT, "profiles", "up_gemm_hbm_traffic.md")
CAL_REPS = 3                # streaming copies of --calibrate-copy-gib each
WEIGHTS_NOTE = {"frag16": "bf16, fragment-block layout (moe_pack_weights once at load, untimed)",
                "rows": "bf16, row-major"}
FP8_NOTE = ("routed experts FP8 E4M3FN with one E8M0 scale per 128x128 block, shared experts "
            "bf16; fragment-block layout (moe_pack_weights once at load, untimed)")


def weights_note(wl, layout):
    return FP8_NOTE if wl.w_dtype == "fp8" else WEIGHTS_NOTE[layout]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


GEMM_SOURCES = ("api.cpp", "common.hpp", "gemm.hip", "launch.hpp")  # define or launch the GEMMs


def source_hash() -> str:
    """Hash of the sources that define and launch the grouped GEMMs, with
    comments and whitespace removed: counters taken on other code do not
    describe the kernels that run now."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        p = os.path.join(ROOT, "fine_grained_sparse_amd", "csrc", name)
        if os.path.exists(p):
            with open(p) as f:
                code = f.read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            h.update(os.path.basename(p).encode())
            h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, layout: str):
    """GB per dispatch of the up-projection for this workload, weight layout
    and kernel source (a row of profiles/up_gemm_hbm_traffic.md), else None."""
    if not os.path.exists(TRAFFIC_MD):
        return None
    want = source_hash()
    with open(TRAFFIC_MD) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 10 and cells[0] == workload and cells[1] == layout and cells[3] == want:
                try:
                    return float(cells[9])
                except ValueError:
                    return None
    return None


def up_kernel(wl, layout):
    """The kernel the library runs for the up projection of this workload."""
    big_rows = wl.T * wl.K >= 64 * wl.E and wl.act_dtype == "bf16"
    if wl.w_dtype == "fp8":
        return ("k_gemm_wide FP8 (" + ("128x512" if big_rows else "16x512") +
                ", register-fed, codes converted to bf16 in registers; the shared expert's "
                "tiles take the bf16 path in the same launch)")
    if big_rows and layout == "frag16":
        return "k_gemm_wide (128x512, register-fed packed weights)"
    return "k_gemm_big (" + ("128x256" if big_rows else "16x512") + ", weights through LDS)"


def is_up_kernel(name):
    """Kernel name (untruncated) of an up-projection dispatch: the SwiGLU
    instantiation of k_gemm_wide<TC, EPI, NSEG, BM, F8> or of
    k_gemm_big<TC, BM, BN, WM, WN, NST, ROWB, EPI, PK>."""
    m = re.search(r"k_gemm_(wide|big)<([^>]*)>", name)
    if not m:
        return False
    args = m.group(2).replace(" ", "").split(",")
    if m.group(1) == "wide":          # k_gemm_wide<TC, EPI, NSEG, BM, F8>
        return args[1] == "1"
    return args[7] == "1"


def get_workload_light(name):
    from moe_inputs import get_workload
    return get_workload(name)


def work_model(wl, counts):
    """Algorithmic flops and bytes of one forward step and of the
    up-projection kernel (routed rows + shared experts).  Bytes: weights of
    the experts that received
    tokens read once, shared / router / latent weights, x read and out
    written once (temporaries excluded).  Flops: the selected experts'
    SwiGLU, the shared experts, the latent maps; the router counted apart
    (fp32-class)."""
    es = 2 if wl.act_dtype == "bf16" else 4
    din, F, d, T = wl.d_in, wl.F, wl.d, wl.T
    Fsh = wl.n_shared * wl.F_shared
    A = wl.T * wl.K
    touched = int(sum(1 for c in counts if c > 0))
    # routed weights: es bytes per element, or one FP8 byte plus one scale
    # byte per 128 x 128 block
    f8 = wl.w_dtype == "fp8"
    wes = 1 if f8 else es
    sblk = (F // 128) * (din // 128) if f8 else 0
    w_expert = 3 * din * F * wes + 3 * sblk
    flops_routed = 2.0 * A * 3 * din * F
    flops_shared = 2.0 * T * 3 * d * Fsh
    flops_latent = 2.0 * T * d * wl.d_latent * 2
    flops_router = 2.0 * T * d * wl.E
    bytes_step = (touched * w_expert + 3 * d * Fsh * es + wl.E * d * 4 + wl.E * 4
                  + 2 * d * wl.d_latent * es + 2 * T * d * es)

    up = dict(
        flops=2.0 * A * din * 2 * F + 2.0 * T * d * 2 * Fsh,
        bytes=(touched * (2 * F * din * wes + 2 * sblk) + 2 * Fsh * d * es + T * din * es
               + A * F * es + T * Fsh * es))
    return dict(touched=touched, flops_bf16=flops_routed + flops_shared + flops_latent,
                flops_router=flops_router, bytes=bytes_step, up=up)


def _events(torch, n, stream):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:        # create the underlying hipEvents before handing them over
        e.record(stream)
    return evs


def prepare(moe, torch, wl, rows, layout):
    """The weights the layer reads: row-major as generated, or packed once
    (a one-time load step, not part of the timed forward)."""
    if layout == "rows" and wl.w_dtype != "fp8":   # FP8 experts are read packed only
        return rows
    packed = moe.pack_weights(rows, n_shared=wl.n_shared)
    torch.cuda.synchronize()
    return packed


def measure_layer(moe, torch, wl, weights, steps, warmup, seed, layout):
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
    evs = [_events(torch, nev, stream) for _ in range(steps)]
    for _ in range(warmup):
        moe.forward(x, W_r, b, weights, wl.K, wl.scale, **kw)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        moe.forward(x, W_r, b, weights, wl.K, wl.scale, stage_events=evs[i], **kw)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    per_step = sorted(evs[i][0].elapsed_time(evs[i][nev - 1]) for i in range(steps))
    stages = {}
    for j in range(1, nev):
        stages[moe.STAGES[j]] = sum(evs[i][j - 1].elapsed_time(evs[i][j]) for i in range(steps)) / steps
    wm = work_model(wl, counts)
    up_ms = stages["up"]
    up = wm["up"]
    traffic = load_traffic(wl.name, layout)
    kernel = up_kernel(wl, layout)
    if up["flops"] / up["bytes"] >= RIDGE_BF16:
        ach = up["flops"] / (up_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / PEAK_BF16_TFLOPS, 4), traffic=traffic, kernel=kernel,
                    avg_ms=round(up_ms, 4), algorithmic_tflop=round(up["flops"] / 1e12, 4),
                    algorithmic_gb=round(up["bytes"] / 1e9, 3))
    else:
        ach = up["bytes"] / (up_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(ach / PEAK_HBM_GBS, 4), traffic=traffic, kernel=kernel,
                    avg_ms=round(up_ms, 4), algorithmic_gb=round(up["bytes"] / 1e9, 3),
                    algorithmic_tflop=round(up["flops"] / 1e12, 4))
    if traffic is not None:
        roof["traffic_unit"] = "GB per launch"
    layer_s = ms * 1e-3
    layer = dict(tflops_bf16=round(wm["flops_bf16"] / layer_s / 1e12, 2),
                 mfma_frac=round(wm["flops_bf16"] / layer_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                 gbps=round(wm["bytes"] / layer_s / 1e9, 1),
                 hbm_frac=round(wm["bytes"] / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                 algorithmic_tflop=round(wm["flops_bf16"] / 1e12, 4),
                 algorithmic_gb=round(wm["bytes"] / 1e9, 3),
                 touched_experts=wm["touched"],
                 hist_min_mean_max=[min(counts), round(sum(counts) / len(counts), 2), max(counts)])
    return dict(value=wl.T / layer_s, ms=ms, stages={k: round(v, 4) for k, v in stages.items()},
                roofline=roof, layer=layer, inputs=(x, W_r, b),
                median_ms=round(per_step[len(per_step) // 2], 4), min_ms=round(per_step[0], 4))


def measure_router(moe, torch, wl, steps, warmup, seed):
    """moe_router alone: logits (fp32 accumulation of the exact bf16 x bf16
    products of x with the three bf16 planes of W_r), top-K gate, counts.
    Its 70 MB of inputs would stay in the 256 MB MALL between calls, so a
    512 MB buffer is written between timed calls (outside their events)."""
    from moe_inputs import make_router_inputs
    dev = torch.device("cuda:0")
    r_in = make_router_inputs(wl, dev, seed=seed)
    x, W_r, b = r_in["x"], r_in["W_r"], r_in["b"]
    ws = moe.Workspace()
    stream = torch.cuda.current_stream()
    grp = dict(n_group=wl.n_group, topk_group=wl.topk_group)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        moe.router(x, W_r, b, wl.K, wl.scale, workspace=ws, stream=stream, **grp)
    torch.cuda.synchronize()
    evs = [_events(torch, 2, stream) for _ in range(steps)]
    for i in range(steps):
        flush.fill_(i & 255)
        evs[i][0].record(stream)
        moe.router(x, W_r, b, wl.K, wl.scale, workspace=ws, stream=stream, **grp)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ms = sum(per_call) / steps
    del flush
    fl = 2.0 * wl.T * wl.d * wl.E
    ach = fl / (ms * 1e-3) / 1e12
    return dict(value=round(wl.T / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 4),
                median_ms=round(per_call[steps // 2], 4), min_ms=round(per_call[0], 4),
                mall="512 MB written between calls",
                roofline=dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_F32_TFLOPS,
                              unit="TFLOP/s", frac=round(ach / PEAK_F32_TFLOPS, 4), traffic=None,
                              kernel="router logits + top-K gate (fp32-accurate, bf16x3 MFMA)",
                              note="fp32 flops 2*T*d*E against the fp32 matrix peak; executed "
                                   "as 3 bf16 MFMA passes",
                              executed_bf16_tflops=round(3 * ach, 2)),
                config=dict(workload=wl.name, T=wl.T, d=wl.d, E=wl.E, K=wl.K, n_group=wl.n_group,
                            topk_group=wl.topk_group))


def measure_bias_steps(moe, torch, seed):
    """The two bias updates after a batch: the sign step from the K2 prefill
    batch's expert histogram (E = 384, O(E)), and Quantile Balancing over the
    K3 router at 4096 tokens (router logits + a per-expert order statistic)."""
    from moe_inputs import get_workload, make_router_inputs
    dev = torch.device("cuda:0")
    out = {}
    wl = get_workload("k2_prefill_t16384")
    g = torch.Generator(device="cpu").manual_seed(seed)
    counts = torch.randint(0, 2 * wl.T * wl.K // wl.E, (wl.E,), generator=g, dtype=torch.int32).to(dev)
    b = torch.zeros(wl.E, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(10):
        moe.bias_update(counts, b, 1e-3)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(200):
        moe.bias_update(counts, b, 1e-3)
    t1.record(stream)
    torch.cuda.synchronize()
    out["bias_update_e384"] = dict(us_per_call=round(t0.elapsed_time(t1) / 200 * 1e3, 2),
                                   config=dict(E=wl.E, gamma=1e-3))
    wl = get_workload("k3_latent_t4096")
    r = make_router_inputs(wl, dev, seed=seed)
    ws = moe.Workspace()
    for _ in range(3):
        moe.bias_quantile(r["x"], r["W_r"], wl.K, workspace=ws)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(20):
        moe.bias_quantile(r["x"], r["W_r"], wl.K, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / 20
    fl = 2.0 * wl.T * wl.d * wl.E
    out["bias_quantile_k3_t4096"] = dict(
        ms_per_call=round(ms, 4), fp32_tflops=round(fl / (ms * 1e-3) / 1e12, 2),
        frac_of_fp32_peak=round(fl / (ms * 1e-3) / 1e12 / PEAK_F32_TFLOPS, 4),
        config=dict(T=wl.T, d=wl.d, E=wl.E, K=wl.K))
    return out


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

    n, s = run(nth)
    if s < target_s / 2:
        n2 = int(min(wl.T, 96 * nth, max(nth, nth * int(target_s / max(s, 1e-3)))))
        if n2 > n:
            n, s = run(n2)
    return dict(value=round(n / s, 3), unit="tokens/s", cores=nth, kind="oracle",
                sample=(f"{n} random tokens of the {wl.T}-token batch, whole layer per token "
                        f"(router over {wl.E} experts, top-{wl.K}, {wl.K} routed + "
                        f"{wl.n_shared} shared SwiGLU experts), fp64, {s:.1f} s"),
                seconds=round(s, 2))


def summarize_counters(fetch_dir, write_dir, workload, layout, copy_gib):
    """One markdown row of profiles/up_gemm_hbm_traffic.md from two rocprofv3 --pmc passes
    of this script (FETCH_SIZE, then WRITE_SIZE), each run with
    --calibrate-copy-gib so that it also holds CAL_REPS streaming copies
    (torch.neg, fp32) of known size.  Kernel names must not be truncated
    (no -T; see is_up_kernel).  Counter rows of a kernel split into several
    dispatches (the large copy) are summed."""
    def load(d):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as f:
                rows += list(csv.DictReader(f))
        return rows

    if copy_gib <= 0:
        raise SystemExit("--calibrate-copy-gib must name the copy size the passes ran with")
    copy_bytes = CAL_REPS * (int(copy_gib * (1 << 30)) // 4) * 4   # read (= written) by the copies
    out = {}
    for tag, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in load(d) if r["Counter_Name"] == tag]
        up = [float(r["Counter_Value"]) for r in rows if is_up_kernel(r["Kernel_Name"])]
        cal = [float(r["Counter_Value"]) for r in rows if "neg_kernel" in r["Kernel_Name"]]
        if not up or not cal:
            raise SystemExit(f"{tag}: no up-projection dispatches or no copy calibration in {d}")
        scale = copy_bytes / (sum(cal) * 1024)
        out[tag] = (sum(up) / len(up), len(up), scale)
    f_kib, n, f_sc = out["FETCH_SIZE"]
    w_kib, _, w_sc = out["WRITE_SIZE"]
    gb = (f_kib * 1024 * f_sc + w_kib * 1024 * w_sc) / 1e9
    wl = get_workload_light(workload)
    row = (f"| {workload} | {layout} | {up_kernel(wl, layout).split(' ')[0]} | {source_hash()} | {n} | "
           f"{f_kib:.6g} | {w_kib:.6g} | {f_sc:.3f} | {w_sc:.3f} | {gb:.3f} |")
    print(row)
    return row


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k2_prefill_t16384")
    ap.add_argument("--also", default="k2_decode_t256,k2_router_t4096,k2_router_g8_t4096,k3_latent_t4096,"
                                      "k2_decode_fp8_t256,k2_prefill_fp8_t16384",
                    help="comma-separated extra workloads ('' for none)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="target seconds of oracle time (0 skips the CPU baseline)")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--bias-steps", type=int, default=1,
                    help="also time the bias updates (moe_bias_update, moe_bias_quantile); 0 = skip")
    ap.add_argument("--layout", choices=("frag16", "rows"), default="frag16",
                    help="weight layout the layer reads: packed once at load (frag16, "
                         "moe_pack_weights, outside the timed steps) or row-major")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="also run a plain streaming copy (out = -in, fp32) of this many GiB "
                         "three times, to scale HBM byte counters (0 = off)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the profiles/up_gemm_hbm_traffic.md row of --workload from two rocprofv3 "
                         "--pmc output directories and exit (no GPU use)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload, args.layout, args.calibrate_copy_gib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is measured on one GPU's share; the collectives that would shard it are not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fine_grained_sparse_amd as moe
    from moe_inputs import get_workload, make_expert_weights

    if args.calibrate_copy_gib > 0:
        n = int(args.calibrate_copy_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(CAL_REPS):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {CAL_REPS} x (read {n * 4} B, write {n * 4} B)")
        del src, dst
        torch.cuda.empty_cache()
    wl = get_workload(args.workload)
    if wl.router_only:
        sys.exit("choose a whole-layer workload")
    log(f"[bench] generating weights for {wl.name} on the GPU")
    rows = make_expert_weights(wl, "cuda:0", seed=args.seed)
    weights = prepare(moe, torch, wl, rows, args.layout)
    if args.cpu_baseline_seconds <= 0:
        del rows
        rows = None
    torch.cuda.synchronize()
    log(f"[bench] timing {wl.name}: warmup {args.warmup}, steps {args.steps}")
    main_r = measure_layer(moe, torch, wl, weights, args.steps, args.warmup, args.seed, args.layout)
    log(f"[bench] {wl.name}: {main_r['ms']:.3f} ms/step, stages {main_r['stages']}")
    main_wl = wl
    also = {}
    others = [s for s in args.also.split(",") if s]
    for name in others:
        awl = get_workload(name)
        log(f"[bench] timing {name}")
        if awl.router_only:
            r = measure_router(moe, torch, awl, max(args.steps, 100), args.warmup, args.seed)
            log(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step")
            also[name] = r
            continue
        same = (awl.d, awl.E, awl.F, awl.n_shared, awl.F_shared, awl.d_latent, awl.act_dtype, awl.w_dtype) == \
               (wl.d, wl.E, wl.F, wl.n_shared, wl.F_shared, wl.d_latent, wl.act_dtype, wl.w_dtype)
        if not same:
            del weights
            torch.cuda.empty_cache()
            log(f"[bench] generating weights for {name} on the GPU")
            weights = prepare(moe, torch, awl, make_expert_weights(awl, "cuda:0", seed=args.seed),
                              args.layout)
            wl = awl
        n_steps = max(args.steps, 50 if awl.T <= 1024 else 20)   # decode-sized: more, shorter steps
        r = measure_layer(moe, torch, awl, weights, n_steps, args.warmup, args.seed, args.layout)
        log(f"[bench] {name}: {r['ms']:.3f} ms/step, stages {r['stages']}")
        also[name] = dict(value=round(r["value"], 1), unit="tokens/s", ms_per_step=round(r["ms"], 4),
                          median_ms=r["median_ms"], min_ms=r["min_ms"],
                          roofline=r["roofline"], layer=r["layer"], stages_ms=r["stages"],
                          config=dict(workload=name, T=awl.T, d=awl.d, E=awl.E, K=awl.K,
                                      F=awl.F, n_shared=awl.n_shared, F_shared=awl.F_shared,
                                      d_latent=awl.d_latent, scale=awl.scale,
                                      weights=weights_note(awl, args.layout)))
    if args.bias_steps:
        log("[bench] bias updates")
        del weights
        torch.cuda.empty_cache()
        also.update(measure_bias_steps(moe, torch, args.seed))
        log(f"[bench] bias: {also['bias_update_e384']['us_per_call']} us (sign), "
            f"{also['bias_quantile_k3_t4096']['ms_per_call']} ms (quantile)")
    # The oracle runs last: its host copies of the experts (tens of GB) and
    # threads must not share the host with any GPU timing.
    cpu = None
    if args.cpu_baseline_seconds > 0:
        log("[bench] CPU baseline (oracle)")
        x, W_r, b = main_r["inputs"]
        cpu = cpu_baseline(torch, main_wl, rows, x, W_r, b, args.cpu_baseline_seconds, args.seed)
        log(f"[bench] oracle: {cpu['value']} tokens/s on {cpu['cores']} threads")
    rows = None
    mw = get_workload(args.workload)
    line = {
        "metric": METRIC, "value": round(main_r["value"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_r["ms"], 4),
        "median_ms": main_r["median_ms"], "min_ms": main_r["min_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": mw.act_dtype,
        "data": "synthetic (seeded N(0,1) x, N(0,1/fan_in) weights, Zipf(1.1) expert skew)",
        "config": dict(workload=mw.name, T=mw.T, d=mw.d, E=mw.E, K=mw.K, F=mw.F,
                       n_shared=mw.n_shared, F_shared=mw.F_shared, d_latent=mw.d_latent,
                       scale=mw.scale, weights=weights_note(mw, args.layout),
                       parallelism="single-gpu"),
        "roofline": main_r["roofline"], "cpu_baseline": cpu, "layer": main_r["layer"],
        "stages_ms": main_r["stages"], "kernel_source": source_hash(), "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
