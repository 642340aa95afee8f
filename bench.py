#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

A step is one moe_forward call (router, top-K gate, dispatch, SwiGLU
experts, combine with the shared expert) over one batch of seeded synthetic
input already resident in HBM.  Prints ONE JSON line.

Default workload: the K2-shaped layer at 16384 tokens (prefill-sized
grouped GEMMs).  Measured in the same run and reported under "also": the
256-token decode batch on the same weights, the same prefill batch with a
stronger expert skew, the router alone at 4096 tokens, the K3-shaped latent
layer, the FP8 layers and the bias updates.
Per-stage durations come from hipEvents the library records at its stage
boundaries on the launch stream (include/moe.h, MOE_EV_*); the up, down and
combine stages are one kernel each.  "roofline" describes the up projection
(the grouped SwiGLU GEMM, the dominant kernel); "kernels" gives the same for
the down projection and the combine.  Each "traffic" is read from
profiles/hbm_traffic.md when that table holds a row for the workload and
stage taken with the current kernel sources (otherwise null);
`--summarize-counters` writes such rows from two rocprofv3 --pmc passes
(FETCH_SIZE, WRITE_SIZE) of this script, `--summarize-sq` the rows of
profiles/sq_counters.md (MFMA busy, shader clock) from one pass.
The "yardsticks" leg measures, in the same run, a pure HBM streaming read and
a register-only bf16 MFMA loop (with the shader clock it ran at); each
roofline is also given as a fraction of those measured peaks.
Other modes, each printing its own JSON line instead: `--sweep T1,T2,...`
(the layer over batch sizes) and `--ep G` (one GPU's share under G-way
expert parallelism: each slice of E/G experts through moe_forward_slice
under the layer's own routing, beside the whole layer on one GPU).
"""
import argparse
import dataclasses
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
TRAFFIC_MD = os.path.join(ROOT, "profiles", "hbm_traffic.md")
SQ_MD = os.path.join(ROOT, "profiles", "sq_counters.md")
CAL_REPS = 3                # streaming copies of --calibrate-copy-gib each
WEIGHTS_NOTE = {"frag16": "bf16, fragment-block layout (moe_pack_weights once at load, untimed)",
                "rows": "bf16, row-major"}
FP8_NOTE = ("routed experts FP8 E4M3FN with one E8M0 scale per 128x128 block, shared experts "
            "bf16; fragment-block layout (moe_pack_weights once at load, untimed)")
# the library's sources that define or launch the layer's kernels
LAYER_SOURCES = ("api.cpp", "common.hpp", "launch.hpp", "gemm.hip", "router.hip", "dispatch.hip")


def weights_note(wl, layout):
    if wl.w_dtype == "f32":
        return "fp32, row-major (the fp32 layer has no packed layout)"
    return FP8_NOTE if wl.w_dtype == "fp8" else WEIGHTS_NOTE[layout]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the sources that define and launch the layer's kernels, with
    comments and whitespace removed: counters taken on other code do not
    describe the kernels that run now."""
    h = hashlib.sha256()
    for name in LAYER_SOURCES:
        p = os.path.join(ROOT, "fine_grained_sparse_amd", "csrc", name)
        if os.path.exists(p):
            with open(p) as f:
                code = f.read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            h.update(os.path.basename(p).encode())
            h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def _md_rows(path):
    if not os.path.exists(path):
        return []
    rows = []
    with open(path) as f:
        for line in f:
            if line.startswith("|") and not line.startswith("|---"):
                rows.append([c.strip() for c in line.strip().strip("|").split("|")])
    return rows


def load_traffic(workload: str, layout: str, stage: str):
    """HBM-side GB per launch of one stage's kernel for this workload, weight
    layout and kernel source (a row of profiles/hbm_traffic.md), else None."""
    want = source_hash()
    for c in _md_rows(TRAFFIC_MD):
        if len(c) >= 11 and c[0] == workload and c[1] == layout and c[2] == stage and c[4] == want:
            try:
                return float(c[10])
            except ValueError:
                return None
    return None


def up_kernel(wl, layout):
    """The kernel the library runs for the up projection of this workload."""
    big_rows = wl.T * wl.K >= 10 * wl.E and wl.act_dtype == "bf16"  # the planner's switch
    if wl.w_dtype == "f32":
        return "k_gemm (fp32, 16 x 256 register-staged tiles)"
    if wl.w_dtype == "fp8":
        return ("k_gemm_wide FP8 (" + ("128x512" if big_rows else "16x512") +
                ", register-fed, codes converted to bf16 in registers; the shared expert's "
                "tiles take the bf16 path in the same launch)")
    if big_rows and layout == "frag16":
        return "k_gemm_wide (128x512, register-fed packed weights)"
    return "k_gemm_big (" + ("128x256" if big_rows else "16x512") + ", weights through LDS)"


def gemm_epilogue(name):
    """1 for the SwiGLU instantiation of a GEMM kernel (k_gemm_wide<TC, EPI,
    NSEG, BM, F8>, k_gemm_big<TC, BM, BN, WM, WN, NST, ROWB, EPI, PK>,
    k_gemm<TC, EPI, ...>), 0 for the store epilogue, None if not a GEMM."""
    m = re.search(r"k_gemm(_wide|_big)?<([^>]*)>", name)
    if not m:
        return None
    args = m.group(2).replace(" ", "").split(",")
    if m.group(1) == "_wide":
        return int(args[1] == "1")
    if m.group(1) == "_big":
        return int(args[7] == "1")
    return int(args[1] == "1")


def label_stages(dispatches):
    """Stage of every dispatch of the layer's kernels, in dispatch order.
    dispatches: [(dispatch id, kernel name)].  A forward call starts with
    k_split3; its GEMMs come in the order router logits, [x_lat], up (the
    SwiGLU one), down, [latent output map]; the rest are named by their
    kernel."""
    out = {}
    phase = None          # None, "router", "up", "combine": the last landmark of the call
    for did, name in sorted(dispatches):
        epi = gemm_epilogue(name)
        if "k_split3" in name:
            stage, phase = "split", None
        elif "k_topk_gate" in name:
            stage = "gate"
        elif "k_dispatch" in name:
            stage = "dispatch"
        elif "k_combine" in name:
            stage, phase = "combine", "combine"
        elif epi == 1:
            stage, phase = "up", "up"
        elif epi == 0:
            if phase is None:
                stage, phase = "router", "router"
            elif phase == "router":
                stage = "latent"
            elif phase == "up":
                stage, phase = "down", "down"
            elif phase == "combine":
                stage = "end"
            else:
                continue
        else:
            continue
        out[did] = stage
    return out


def get_workload_light(name):
    from moe_inputs import get_workload
    return get_workload(name)


def work_model(wl, counts):
    """Algorithmic flops and bytes of one forward step and of the up, down,
    combine and (latent form) output-map kernels.  Bytes: weights of the
    experts that received tokens read once, shared / router / latent
    weights, x read and out written once; a kernel's own inputs and outputs
    (H, Y) count for that kernel only.  Flops: the selected experts' SwiGLU,
    the shared experts, the latent maps; the router counted apart
    (fp32-class)."""
    es = 2 if wl.act_dtype == "bf16" else 4
    din, F, d, T, dl = wl.d_in, wl.F, wl.d, wl.T, wl.d_latent
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
    flops_latent = 2.0 * T * d * dl * 2
    flops_router = 2.0 * T * d * wl.E
    bytes_step = (touched * w_expert + 3 * d * Fsh * es + wl.E * d * 4 + wl.E * 4
                  + 2 * d * dl * es + 2 * T * d * es)
    x_in = T * d * es + (T * dl * es if dl else 0)      # x (and x_lat) read once
    up = dict(flops=2.0 * A * din * 2 * F + 2.0 * T * d * 2 * Fsh,
              bytes=(touched * (2 * F * din * wes + 2 * sblk) + 2 * Fsh * d * es + x_in
                     + A * F * es + T * Fsh * es))
    if dl:   # routed experts only; the shared down projection is part of the output map
        down = dict(flops=2.0 * A * F * din,
                    bytes=touched * (din * F * wes + sblk) + A * F * es + A * din * es)
        combine = dict(flops=2.0 * A * din, bytes=A * din * es + A * 8 + T * din * es)
        end = dict(flops=2.0 * T * (Fsh + dl) * d,
                   bytes=(Fsh + dl) * d * es + T * (Fsh + dl) * es + T * d * es)
    else:
        down = dict(flops=2.0 * A * F * d + 2.0 * T * Fsh * d,
                    bytes=(touched * (d * F * wes + sblk) + Fsh * d * es + A * F * es
                           + T * Fsh * es + (A + (T if Fsh else 0)) * d * es))
        combine = dict(flops=2.0 * A * d,
                       bytes=(A + (T if Fsh else 0)) * d * es + A * 8 + T * d * es)
        end = None
    return dict(touched=touched, flops_bf16=flops_routed + flops_shared + flops_latent,
                flops_router=flops_router, bytes=bytes_step, up=up, down=down, combine=combine,
                end=end)


def roofline(work, ms, kernel, traffic, ys=None):
    """Roofline object of one kernel: algorithmic work per launch over its
    average duration, against the spec peak of the bound its intensity
    selects (and against the peak measured in this run, when known)."""
    mfma = work["flops"] / work["bytes"] >= RIDGE_BF16
    if mfma:
        ach = work["flops"] / (ms * 1e-3) / 1e12
        r = dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                 frac=round(ach / PEAK_BF16_TFLOPS, 4))
    else:
        ach = work["bytes"] / (ms * 1e-3) / 1e9
        r = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                 frac=round(ach / PEAK_HBM_GBS, 4))
    r.update(traffic=traffic, kernel=kernel, avg_ms=round(ms, 4),
             algorithmic_tflop=round(work["flops"] / 1e12, 4),
             algorithmic_gb=round(work["bytes"] / 1e9, 3))
    if traffic is not None:
        r["traffic_unit"] = "GB per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    if ys:
        key = "mfma_tflops" if mfma else "hbm_read_gbs"
        r["measured_peak"] = ys[key]
        r["frac_of_measured"] = round(ach / ys[key], 4)
    return r


def _events(torch, n, stream):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:        # create the underlying hipEvents before handing them over
        e.record(stream)
    return evs


def prepare(moe, torch, wl, rows, layout):
    """The weights the layer reads: row-major as generated, or packed once
    (a one-time load step, not part of the timed forward)."""
    if (layout == "rows" and wl.w_dtype != "fp8") or wl.w_dtype == "f32":
        return rows                  # FP8 experts are read packed only; fp32 row-major only
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
                wm=wm, layer=layer, inputs=(x, W_r, b),
                median_ms=round(per_step[len(per_step) // 2], 4), min_ms=round(per_step[0], 4))


def measure_slices(moe, torch, wl, weights, G, steps, warmup, seed):
    """One GPU's share of the layer under G-way expert parallelism (E/G
    experts per GPU), for each of the G slices: moe_forward_slice over the
    layer's own routing of all T tokens, as if each GPU had received the
    rows routed to its experts.  Routed experts only: the router and the
    shared experts would run on each token's owner, and the all-to-all
    exchange is not built.  Returns one dict per slice: its rows, touched
    experts, time and algorithmic rates."""
    from moe_inputs import make_router_inputs
    dev = torch.device("cuda:0")
    r_in = make_router_inputs(wl, dev, seed=seed)
    x, W_r, b = r_in["x"], r_in["W_r"], r_in["b"]
    idx, w, counts = moe.router(x, W_r, b, wl.K, wl.scale)
    counts = counts.cpu().tolist()
    out = torch.empty((wl.T, wl.d), dtype=x.dtype, device=dev)
    ws = moe.Workspace()
    stream = torch.cuda.current_stream()
    f8 = wl.w_dtype == "fp8"
    wes = 1 if f8 else (2 if wl.act_dtype == "bf16" else 4)
    sblk = (wl.F // 128) * (wl.d_in // 128) if f8 else 0
    per = wl.E // G
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = []
    for g in range(G):
        e0, e1 = g * per, (g + 1) * per
        sw = {k: weights[k][e0:e1] for k in ("W_gate", "W_up", "W_down") + moe.SCALE_NAMES
              if weights.get(k) is not None}
        if "layout" in weights:
            sw["layout"] = weights["layout"]
        for _ in range(warmup):
            moe.forward_slice(x, idx, w, sw, e0, wl.E, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(steps):
            moe.forward_slice(x, idx, w, sw, e0, wl.E, out=out, workspace=ws, stream=stream)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        rows = int(sum(counts[e0:e1]))
        touched = int(sum(1 for c in counts[e0:e1] if c > 0))
        flops = 2.0 * rows * 3 * wl.d_in * wl.F
        wbytes = touched * (3 * wl.d_in * wl.F * wes + 3 * sblk)
        res.append(dict(experts=[e0, e1], rows=rows, touched=touched, ms=round(ms, 4),
                        tflops=round(flops / (ms * 1e-3) / 1e12, 1),
                        weight_gbps=round(wbytes / (ms * 1e-3) / 1e9, 1)))
        log(f"[bench] slice {e0}..{e1 - 1}: {rows} rows, {touched} experts touched, {ms:.3f} ms")
    return res


def kernel_rooflines(wl, r, layout, ys):
    """Rooflines of the up projection (the dominant kernel) and of the down
    projection and the combine, from the stage events of the timed steps.
    In the latent form the combine stage also holds the output map
    [Hs | R] [Ws_down | W_lat_up]^T, so its roofline is that of the pair."""
    wm, st = r["wm"], r["stages"]
    up = roofline(wm["up"], st["up"], up_kernel(wl, layout), load_traffic(wl.name, layout, "up"), ys)
    down = roofline(wm["down"], st["down"], up_kernel(wl, layout).split(" ")[0] + " (store epilogue)",
                    load_traffic(wl.name, layout, "down"), ys)
    if wm["end"] is None:
        comb = roofline(wm["combine"], st["end"], "k_combine (gather, fp32 sum, one bf16 rounding)",
                        load_traffic(wl.name, layout, "combine"), ys)
    else:
        both = dict(flops=wm["combine"]["flops"] + wm["end"]["flops"],
                    bytes=wm["combine"]["bytes"] + wm["end"]["bytes"])
        comb = roofline(both, st["end"], "k_combine (latent weighted sum) + output map GEMM", None, ys)
    return up, dict(down=down, combine=comb)


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
    res = dict(value=round(wl.T / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 4),
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
    return res, (x, W_r, b)


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


def gpu_clocks(torch):
    """Current shader (SCLK) and memory (MCLK) clocks of the GPU in MHz: the
    sysfs DPM tables (the level marked '*') of the card whose PCI bus matches
    device 0, else amd-smi's clock metrics.  A snapshot between timings, not
    the clock under load (the MFMA yardstick and the counter tables give
    that)."""
    import subprocess

    def dpm(path):
        try:
            with open(path) as f:
                for ln in f:
                    if ln.rstrip().endswith("*"):
                        return int("".join(ch for ch in ln.split(":")[1] if ch.isdigit()))
        except (OSError, ValueError, IndexError):
            return None
        return None

    bus = None
    try:
        pr = torch.cuda.get_device_properties(0)
        if getattr(pr, "pci_bus_id", None) is not None:
            bus = "%02x:%02x" % (pr.pci_bus_id, getattr(pr, "pci_device_id", 0))
    except Exception:
        pass
    cards = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        sclk, mclk = dpm(dev + "/pp_dpm_sclk"), dpm(dev + "/pp_dpm_mclk")
        if sclk is None and mclk is None:
            continue
        cards.append((os.path.basename(os.path.realpath(dev)), sclk, mclk))
    if cards:
        pick = [c for c in cards if bus and bus in c[0]] or (cards if len(cards) == 1 else [])
        if pick:
            return dict(sclk_mhz=pick[0][1], mclk_mhz=pick[0][2], source="sysfs pp_dpm (" + pick[0][0] + ")")
    try:
        out = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True, text=True,
                             timeout=30).stdout
        data = json.loads(out[out.index("["):] if "[" in out else out)
        ent = data[0] if isinstance(data, list) else data
        clk = ent.get("clock", ent)

        def mhz(v):
            v = v.get("clk", v) if isinstance(v, dict) else v
            v = v.get("value") if isinstance(v, dict) else v
            try:
                return int(float(v))
            except (TypeError, ValueError):
                return None
        gfx = [mhz(v) for k, v in clk.items() if k.startswith("gfx")]
        mem = [mhz(v) for k, v in clk.items() if k.startswith("mem")]
        gfx = [g for g in gfx if g is not None]
        mem = [m for m in mem if m is not None]
        return dict(sclk_mhz=max(gfx) if gfx else None, mclk_mhz=max(mem) if mem else None,
                    source="amd-smi metric --clock")
    except Exception as e:  # no sysfs table and no usable amd-smi: say so
        return dict(sclk_mhz=None, mclk_mhz=None, source=f"unavailable ({type(e).__name__})")


def yardsticks(torch, read_gib=8.0, mfma_ms=20.0):
    """Measured peaks of this GPU in this run (libyardstick.so): the best of
    a plain and a non-temporal streaming read of read_gib GiB over a few grid
    sizes, and the register-only bf16 MFMA loop on one workgroup (4 waves)
    per CU, with the shader clock it ran at (clock64 over wall_clock64)."""
    import ctypes
    path = os.path.join(ROOT, "fine_grained_sparse_amd", "libyardstick.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build with fine_grained_sparse_amd/build.py")
    L = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.ys_stream_read.argtypes = [vp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    L.ys_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
    L.ys_mfma_flops_per_block_iter.restype = i64
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    s = ctypes.c_void_p(stream.cuda_stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        best = None
        for _ in range(reps):
            t0.record(stream)
            rc = fn()
            t1.record(stream)
            if rc:
                raise RuntimeError(f"yardstick launch failed: hipError {rc}")
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1)
            best = ms if best is None else min(best, ms)
        return best

    nbytes = int(read_gib * (1 << 30)) // 16 * 16
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    reads = {}
    for nt in (0, 1):
        for inflight in (8, 16):
            for blocks in (512, 1024, 2048, 4096):
                sink = torch.empty(blocks * 512, dtype=torch.int32, device=dev)
                ms = timed(lambda: L.ys_stream_read(buf.data_ptr(), nbytes, nt, inflight, blocks,
                                                    sink.data_ptr(), s), 4)
                key = f"{'nt' if nt else 'plain'}_x{inflight}_{blocks}"
                reads[key] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, sink
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    per_iter = L.ys_mfma_flops_per_block_iter() * cus
    sink = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(cus * 4, dtype=torch.int64, device=dev)
    ms1 = timed(lambda: L.ys_mfma_loop(1000, cus, sink.data_ptr(), clocks.data_ptr(), s), 2)
    iters = max(1000, int(1000 * mfma_ms / max(ms1, 1e-3)))
    ms = timed(lambda: L.ys_mfma_loop(iters, cus, sink.data_ptr(), clocks.data_ptr(), s), 3)
    c = clocks.view(cus, 4).cpu().double()
    khz = ctypes.CDLL(path).ys_wall_clock_khz()
    ghz = ((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * khz / 1e6).median().item() if khz else None
    best_key = max(reads, key=reads.get)
    return dict(hbm_read_gbs=reads[best_key], hbm_read_best=best_key, hbm_read_all=reads,
                mfma_tflops=round(per_iter * iters / (ms * 1e-3) / 1e12, 1),
                mfma_clock_ghz=round(ghz, 3) if ghz else None, mfma_blocks=cus, mfma_iters=iters,
                note=("HBM: one read of an 8 GiB buffer, 16 B per lane, 8 or 16 loads in flight, "
                      "best of the sweep; MFMA: "
                      "v_mfma_f32_16x16x32_bf16 chains on registers, one 4-wave workgroup per CU; "
                      "clock = clock64 / wall_clock64 over the loop (median of the workgroups)"))


def host_weights(weights):
    """Host copies of a layer's weights for the oracle (one copy per tensor)."""
    return {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in weights.items()
            if k in ("W_gate", "W_up", "W_down", "Ws_gate", "Ws_up", "Ws_down", "W_lat_down",
                     "W_lat_up", "W_gate_scale", "W_up_scale", "W_down_scale")}


def _oracle_layer(oracle, wl, hw, W_r, b):
    per = {k: ([hw[k][e] for e in range(wl.E)] if hw.get(k) is not None else None)
           for k in ("W_gate", "W_up", "W_down", "W_gate_scale", "W_up_scale", "W_down_scale")}
    return oracle.Layer(d=wl.d, E=wl.E, K=wl.K, F=wl.F, scale=wl.scale, W_r=W_r, b=b,
                        W_gate=per["W_gate"], W_up=per["W_up"], W_down=per["W_down"],
                        W_gate_scale=per["W_gate_scale"], W_up_scale=per["W_up_scale"],
                        W_down_scale=per["W_down_scale"], n_shared=wl.n_shared,
                        F_shared=wl.F_shared, Ws_gate=hw.get("Ws_gate"), Ws_up=hw.get("Ws_up"),
                        Ws_down=hw.get("Ws_down"), d_latent=wl.d_latent,
                        W_lat_down=hw.get("W_lat_down"), W_lat_up=hw.get("W_lat_up"))


def cpu_baseline(wl, hw, inputs, target_s, seed, full=False, router_only=False):
    """The oracle as it stands (plain fp64 loops, OpenMP over tokens) on the
    host's cores: the whole layer (router over all experts, top-K, K routed
    + the shared SwiGLU experts, latent maps), or the router alone.
    full: every token of the batch through the whole layer.  Otherwise the
    router and the dispatch run over every token, and the expert part
    (oracle_forward_given_routing under that routing) over a random token
    sample sized to about target_s seconds; rows are independent there, so
    the batch's expert time is the sample's per-token time times T.  The
    layer's time is the sum, labelled extrapolated."""
    import numpy as np
    import oracle
    nth = oracle.default_threads()
    x, W_r, b = (t.cpu() for t in inputs)
    info = dict(unit="tokens/s", cores=nth, host_cores=oracle.host_cores(),
                cpu_model=oracle.cpu_model(), kind="oracle")
    if router_only:
        t = time.perf_counter()
        oracle.router(x, W_r, b, wl.K, wl.scale, nthreads=nth)
        sec = time.perf_counter() - t
        return dict(value=round(wl.T / sec, 1), seconds=round(sec, 2), **info,
                    sample=f"all {wl.T} tokens (router over {wl.E} experts, top-{wl.K}), fp64")
    lay = _oracle_layer(oracle, wl, hw, W_r, b)
    what = (f"router over {wl.E} experts, top-{wl.K}, {wl.K} routed + {wl.n_shared} shared "
            f"SwiGLU experts{', latent maps' if wl.d_latent else ''}, fp64")
    if full:
        t = time.perf_counter()
        oracle.forward(lay, x, nthreads=nth)
        sec = time.perf_counter() - t
        return dict(value=round(wl.T / sec, 2), seconds=round(sec, 2), **info,
                    sample=f"all {wl.T} tokens of the batch, whole layer per token ({what})")
    t = time.perf_counter()
    rt = oracle.router(x, W_r, b, wl.K, wl.scale, nthreads=nth)
    router_s = time.perf_counter() - t
    t = time.perf_counter()
    oracle.dispatch(rt["idx"], wl.E)
    dispatch_s = time.perf_counter() - t
    rng = np.random.default_rng(seed)

    def run(n):
        toks = np.sort(rng.choice(wl.T, size=min(n, wl.T), replace=False))
        t = time.perf_counter()
        oracle.forward_given_routing(lay, x[toks].contiguous(), rt["idx"][toks], rt["w"][toks], nthreads=nth)
        return len(toks), time.perf_counter() - t

    n, sec = run(nth)
    if sec < target_s / 2:
        n2 = int(min(wl.T, max(nth, nth * int(target_s / max(sec, 1e-3)))))
        if n2 > n:
            n, sec = run(n2)
    experts_s = sec / n * wl.T
    layer_s = router_s + dispatch_s + experts_s
    return dict(value=round(wl.T / layer_s, 3), seconds=round(router_s + dispatch_s + sec, 2),
                extrapolated=True, full_batch_s=round(layer_s, 1), router_s=round(router_s, 2),
                dispatch_s=round(dispatch_s, 3), experts_s_extrapolated=round(experts_s, 1), **info,
                sample=(f"router ({wl.E} experts, top-{wl.K}) and dispatch over all {wl.T} tokens; the "
                        f"expert part ({wl.K} routed + {wl.n_shared} shared SwiGLU experts"
                        f"{', latent maps' if wl.d_latent else ''}, fp64) over {n} random tokens under "
                        f"that routing, its per-token time extrapolated to the batch (rows independent)"))


def _load_counter_csv(d):
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows):
    """{dispatch id: dict(name, counters {name: value summed over the rows of
    that dispatch}, start, end)}."""
    out = {}
    for r in rows:
        did = int(r["Dispatch_Id"])
        e = out.setdefault(did, dict(name=r["Kernel_Name"], counters={},
                                     start=int(r.get("Start_Timestamp") or 0),
                                     end=int(r.get("End_Timestamp") or 0)))
        e["counters"][r["Counter_Name"]] = e["counters"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _kernel_short(name):
    m = re.search(r"(k_[a-z0-9_]+)(<[^>]*>)?", name)
    if not m:
        return name
    return (m.group(1) + (m.group(2) or "")).replace("unsigned short", "bf16").replace(" ", "")


def summarize_counters(fetch_dir, write_dir, workload, layout, copy_gib):
    """Rows of profiles/hbm_traffic.md (one per stage kernel of the layer)
    from two rocprofv3 --pmc passes of this script (FETCH_SIZE, then
    WRITE_SIZE), each run with --calibrate-copy-gib so that it also holds
    CAL_REPS streaming copies (torch.neg, fp32) of known size.  The copy's
    counts give the scale of each counter (bytes moved / bytes counted)."""
    if copy_gib <= 0:
        raise SystemExit("--calibrate-copy-gib must name the copy size the passes ran with")
    copy_bytes = CAL_REPS * (int(copy_gib * (1 << 30)) // 4) * 4   # read (= written) by the copies
    per = {}
    for tag, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = _per_dispatch(_load_counter_csv(d))
        cal = sum(v["counters"].get(tag, 0.0) for v in disp.values() if "neg_kernel" in v["name"])
        if not cal:
            raise SystemExit(f"{tag}: no copy calibration dispatches in {d}")
        scale = copy_bytes / (cal * 1024)
        stages = label_stages([(k, v["name"]) for k, v in disp.items() if "neg_kernel" not in v["name"]])
        acc = {}
        for did, st in stages.items():
            acc.setdefault(st, []).append((disp[did]["counters"].get(tag, 0.0), disp[did]["name"]))
        per[tag] = (acc, scale)
    get_workload_light(workload)      # the workload must exist
    rows = []
    f_acc, f_sc = per["FETCH_SIZE"]
    w_acc, w_sc = per["WRITE_SIZE"]
    for stage in ("router", "gate", "dispatch", "latent", "up", "down", "combine", "end"):
        if stage not in f_acc or stage not in w_acc:
            continue
        fv = [v for v, _ in f_acc[stage]]
        wv = [v for v, _ in w_acc[stage]]
        # per launch of the stage: the dispatch stage is four kernels per call
        nk = len({n for _, n in f_acc[stage]})
        f_kib = sum(fv) / len(fv) * nk
        w_kib = sum(wv) / len(wv) * nk
        gb = (f_kib * 1024 * f_sc + w_kib * 1024 * w_sc) / 1e9
        kname = _kernel_short(f_acc[stage][0][1]) if nk == 1 else f"{nk} kernels"
        rows.append(f"| {workload} | {layout} | {stage} | `{kname}` | {source_hash()} | "
                    f"{len(fv) // nk} | {f_kib:.6g} | {w_kib:.6g} | {f_sc:.3f} | {w_sc:.3f} | {gb:.3f} |")
    for r in rows:
        print(r)
    return rows


def summarize_sq(sq_dir, workload, layout):
    """Rows of profiles/sq_counters.md from one rocprofv3 --kernel-trace
    --pmc pass with SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES and
    GRBM_GUI_ACTIVE: per stage kernel, its duration under counter collection,
    cycles per XCD (GRBM_GUI_ACTIVE is summed over the 8 XCDs), the shader
    clock (cycles / duration) and the MFMA busy fraction per SIMD
    (SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x CUs x cycles))."""
    disp = _per_dispatch(_load_counter_csv(sq_dir))
    stages = label_stages([(k, v["name"]) for k, v in disp.items()])
    acc = {}
    for did, st in stages.items():
        acc.setdefault(st, []).append(disp[did])
    rows = []
    for stage in ("router", "latent", "up", "down", "combine", "end"):
        if stage not in acc:
            continue
        ds = acc[stage]
        n = len(ds)
        ms = sum((d["end"] - d["start"]) for d in ds) / n / 1e6
        grbm = sum(d["counters"].get("GRBM_GUI_ACTIVE", 0.0) for d in ds) / n
        mfma = sum(d["counters"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds) / n
        cyc = grbm / 8
        ghz = cyc / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        busy = mfma / (1024 * cyc) if cyc else 0.0
        rows.append(f"| {workload} | {layout} | {stage} | `{_kernel_short(ds[0]['name'])}` | {source_hash()} | "
                    f"{n} | {ms:.3f} | {cyc:.4g} | {ghz:.2f} | {busy:.3f} |")
    for r in rows:
        print(r)
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k2_prefill_t16384")
    ap.add_argument("--also", default="k2_decode_t256,k2_prefill_skew4_t16384,k2_router_t4096,"
                                      "k2_router_g8_t4096,k3_latent_t4096,k2_decode_fp8_t256,"
                                      "k2_prefill_fp8_t16384,tiny_fp32_t128",
                    help="comma-separated extra workloads ('' for none)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0,
                    help="target seconds of oracle time per sampled workload (0 skips the CPU baselines)")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--bias-steps", type=int, default=1,
                    help="also time the bias updates (moe_bias_update, moe_bias_quantile); 0 = skip")
    ap.add_argument("--yardsticks", type=int, default=1,
                    help="measure the HBM read and bf16 MFMA yardsticks in this run (0 = skip)")
    ap.add_argument("--layout", choices=("frag16", "rows"), default="frag16",
                    help="weight layout the layer reads: packed once at load (frag16, "
                         "moe_pack_weights, outside the timed steps) or row-major")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="also run a plain streaming copy (out = -in, fp32) of this many GiB "
                         "three times, to scale HBM byte counters (0 = off)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the profiles/hbm_traffic.md rows of --workload from two rocprofv3 "
                         "--pmc output directories and exit (no GPU use)")
    ap.add_argument("--sweep", metavar="T1,T2,...",
                    help="time --workload's layer at these batch sizes (same weights, seeded inputs "
                         "per size), print one JSON line of the results and exit")
    ap.add_argument("--ep", type=int, default=0, metavar="G",
                    help="time --workload's routed experts as G expert-parallel slices of E/G experts "
                         "(moe_forward_slice under the layer's own routing, K2 form), print one JSON "
                         "line of the results and exit")
    ap.add_argument("--summarize-sq", metavar="SQ_DIR",
                    help="print the profiles/sq_counters.md rows of --workload from one rocprofv3 "
                         "--pmc output directory and exit (no GPU use)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload, args.layout, args.calibrate_copy_gib)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.workload, args.layout)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is measured on one GPU's share; the collectives that would shard it are not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fine_grained_sparse_amd as moe
    from moe_inputs import get_workload, make_expert_weights

    cpu_on = args.cpu_baseline_seconds > 0
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
    if wl.router_only and args.sweep:
        sweep = []
        for T in (int(t) for t in args.sweep.split(",") if t):
            swl = dataclasses.replace(wl, T=T, name=f"{wl.name}@T={T}")
            r, _ = measure_router(moe, torch, swl, max(args.steps, 100), args.warmup, args.seed)
            log(f"[bench] sweep {wl.name} T={T}: {r['ms_per_step']:.4f} ms/step, {r['value']:.0f} tokens/s")
            sweep.append(dict(T=T, ms=r["ms_per_step"], tokens_per_s=r["value"]))
            torch.cuda.empty_cache()
        print(json.dumps(dict(workload=wl.name, steps=max(args.steps, 100), warmup=args.warmup, sweep=sweep)),
              flush=True)
        return
    if wl.router_only:
        sys.exit("choose a whole-layer workload")
    log(f"[bench] generating weights for {wl.name} on the GPU")
    rows = make_expert_weights(wl, "cuda:0", seed=args.seed)
    weights = prepare(moe, torch, wl, rows, args.layout)
    torch.cuda.synchronize()
    if args.ep:
        del rows
        if wl.d_latent or wl.E % args.ep:
            sys.exit("--ep takes a K2-form layer whose experts divide evenly (the latent maps would "
                     "run on each token's owner, outside the slice)")
        full = measure_layer(moe, torch, wl, weights, args.steps, args.warmup, args.seed, args.layout)
        log(f"[bench] {wl.name} on one GPU: {full['ms']:.3f} ms/step, stages {full['stages']}")
        res = measure_slices(moe, torch, wl, weights, args.ep, args.steps, args.warmup, args.seed)
        ms = [r["ms"] for r in res]
        rows = [r["rows"] for r in res]
        print(json.dumps(dict(workload=wl.name, layout=args.layout, ep=args.ep, steps=args.steps,
                              warmup=args.warmup, layer_ms=round(full["ms"], 4), layer_stages=full["stages"],
                              slices=res, slice_ms_max=max(ms), slice_ms_mean=round(sum(ms) / len(ms), 4),
                              slice_ms_sum=round(sum(ms), 4),
                              rows_max_over_mean=round(max(rows) * len(rows) / max(sum(rows), 1), 3))),
              flush=True)
        return
    if args.sweep:
        del rows
        sweep = []
        for T in (int(t) for t in args.sweep.split(",") if t):
            swl = dataclasses.replace(wl, T=T, name=f"{wl.name}@T={T}")
            r = measure_layer(moe, torch, swl, weights, args.steps, args.warmup, args.seed, args.layout)
            line = dict(T=T, ms=round(r["ms"], 4), tokens_per_s=round(r["value"], 1),
                        rows_per_expert=round(T * wl.K / wl.E, 2), stages=r["stages"])
            log(f"[bench] sweep {wl.name} T={T}: {r['ms']:.3f} ms/step, {r['value']:.0f} tokens/s, "
                f"{line['rows_per_expert']} rows per expert")
            sweep.append(line)
            del r
            torch.cuda.empty_cache()
        print(json.dumps(dict(workload=wl.name, layout=args.layout, steps=args.steps, warmup=args.warmup,
                              sweep=sweep)), flush=True)
        return
    clocks_before = gpu_clocks(torch)
    log(f"[bench] clocks before: {clocks_before}")
    log(f"[bench] timing {wl.name}: warmup {args.warmup}, steps {args.steps}")
    main_r = measure_layer(moe, torch, wl, weights, args.steps, args.warmup, args.seed, args.layout)
    log(f"[bench] {wl.name}: {main_r['ms']:.3f} ms/step, stages {main_r['stages']}")
    main_wl = wl
    # host copies for the oracle legs, taken between GPU timings (nothing is timed meanwhile)
    host = {}
    if cpu_on:
        log(f"[bench] host copy of the {wl.name} weights for the oracle")
        host[(wl.d, wl.E, wl.F, wl.d_latent, wl.w_dtype)] = host_weights(rows)
    del rows
    cpu_jobs = [(main_wl.name, main_wl, main_r["inputs"], dict())]
    also, also_raw = {}, {}
    others = [s for s in args.also.split(",") if s]
    for name in others:
        awl = get_workload(name)
        log(f"[bench] timing {name}")
        if awl.router_only:
            r, inputs = measure_router(moe, torch, awl, max(args.steps, 100), args.warmup, args.seed)
            log(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step")
            also[name] = r
            if cpu_on and awl.n_group <= 1:
                cpu_jobs.append((name, awl, inputs, dict(router_only=True)))
            continue
        same = (awl.d, awl.E, awl.F, awl.n_shared, awl.F_shared, awl.d_latent, awl.act_dtype, awl.w_dtype) == \
               (wl.d, wl.E, wl.F, wl.n_shared, wl.F_shared, wl.d_latent, wl.act_dtype, wl.w_dtype)
        if not same:
            del weights
            torch.cuda.empty_cache()
            log(f"[bench] generating weights for {name} on the GPU")
            arows = make_expert_weights(awl, "cuda:0", seed=args.seed)
            weights = prepare(moe, torch, awl, arows, args.layout)
            key = (awl.d, awl.E, awl.F, awl.d_latent, awl.w_dtype)
            if cpu_on and (awl.d_latent or awl.w_dtype == "f32") and key not in host:
                log(f"[bench] host copy of the {name} weights for the oracle")
                host[key] = host_weights(arows)
            del arows
            wl = awl
        n_steps = max(args.steps, 50 if awl.T <= 1024 else 20)   # decode-sized: more, shorter steps
        r = measure_layer(moe, torch, awl, weights, n_steps, args.warmup, args.seed, args.layout)
        log(f"[bench] {name}: {r['ms']:.3f} ms/step, stages {r['stages']}")
        also_raw[name] = (awl, r)
        also[name] = dict(value=round(r["value"], 1), unit="tokens/s", ms_per_step=round(r["ms"], 4),
                          median_ms=r["median_ms"], min_ms=r["min_ms"], layer=r["layer"],
                          stages_ms=r["stages"],
                          config=dict(workload=name, T=awl.T, d=awl.d, E=awl.E, K=awl.K,
                                      F=awl.F, n_shared=awl.n_shared, F_shared=awl.F_shared,
                                      d_latent=awl.d_latent, scale=awl.scale,
                                      zipf_scale=awl.zipf_scale if awl.zipf_skew else None,
                                      weights=weights_note(awl, args.layout)))
        if cpu_on and awl.w_dtype != "fp8" and name in ("k2_decode_t256", "k3_latent_t4096", "tiny_fp32_t128"):
            cpu_jobs.append((name, awl, r["inputs"], dict(full=awl.T <= 256)))
    del weights
    torch.cuda.empty_cache()
    if args.bias_steps:
        log("[bench] bias updates")
        also.update(measure_bias_steps(moe, torch, args.seed))
        log(f"[bench] bias: {also['bias_update_e384']['us_per_call']} us (sign), "
            f"{also['bias_quantile_k3_t4096']['ms_per_call']} ms (quantile)")
    ys = None
    if args.yardsticks:
        log("[bench] yardsticks: HBM streaming read, bf16 MFMA loop")
        ys = yardsticks(torch)
        log(f"[bench] yardsticks: {ys['hbm_read_gbs']} GB/s ({ys['hbm_read_best']}), "
            f"{ys['mfma_tflops']} TFLOP/s at {ys['mfma_clock_ghz']} GHz")
    clocks_after = gpu_clocks(torch)
    log(f"[bench] clocks after: {clocks_after}")
    main_roof, main_kernels = kernel_rooflines(main_wl, main_r, args.layout, ys)
    for name, (awl, r) in also_raw.items():
        roof, kern = kernel_rooflines(awl, r, args.layout, ys)
        also[name]["roofline"] = roof
        also[name]["kernels"] = kern
    # The oracle runs last: its host copies of the experts and its threads
    # must not share the host with any GPU timing.
    cpu = None
    for name, jwl, inputs, kw in cpu_jobs:
        hw = None
        if not kw.get("router_only"):
            hw = host.get((jwl.d, jwl.E, jwl.F, jwl.d_latent, jwl.w_dtype))
            if hw is None:
                continue
        log(f"[bench] CPU baseline (oracle): {name}")
        res = cpu_baseline(jwl, hw, inputs, args.cpu_baseline_seconds, args.seed, **kw)
        log(f"[bench] oracle {name}: {res['value']} tokens/s on {res['cores']} threads ({res['seconds']} s)")
        if name == main_wl.name:
            cpu = res
        else:
            also[name]["cpu_baseline"] = res
    host = None
    mw = main_wl
    line = {
        "metric": METRIC, "value": round(main_r["value"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_r["ms"], 4),
        "median_ms": main_r["median_ms"], "min_ms": main_r["min_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": mw.act_dtype,
        "data": "synthetic (seeded N(0,1) x, N(0,1/fan_in) weights, Zipf(1.1) expert skew)",
        "config": dict(workload=mw.name, T=mw.T, d=mw.d, E=mw.E, K=mw.K, F=mw.F,
                       n_shared=mw.n_shared, F_shared=mw.F_shared, d_latent=mw.d_latent,
                       scale=mw.scale, zipf_scale=mw.zipf_scale,
                       weights=weights_note(mw, args.layout), parallelism="single-gpu"),
        "roofline": main_roof, "cpu_baseline": cpu, "kernels": main_kernels,
        "layer": main_r["layer"], "stages_ms": main_r["stages"], "yardsticks": ys,
        "clocks": dict(before=clocks_before, after=clocks_after),
        "kernel_source": source_hash(), "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
