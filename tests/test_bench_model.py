"""Host logic of bench.py (no GPU): the algorithmic work that every roofline
divides by a measured time, the roofline arithmetic itself, the assignment
of profiled dispatches to stages, the source hash that keys the counter
tables, and the clock snapshot.

The expected work is written out here from the layer's shapes (the K2 and
K3 workloads of moe_inputs), term by term, so that a dropped or doubled
term in bench.work_model fails: per token and selected expert a SwiGLU
expert is three d_in x F products, 2 flops per multiply-add; a touched
expert's weights are read once."""
import os
import shutil

import pytest

import bench
from moe_inputs import get_workload

TF = 1e12
GB = 1e9


def _counts(E, A, touched):
    """A histogram of A assignments over the first `touched` experts."""
    c = [0] * E
    for i in range(A):
        c[i % touched] += 1
    return c


def test_k2_prefill_step_work():
    wl = get_workload("k2_prefill_t16384")
    d, F, T, E = 7168, 2048, 16384, 384
    A = T * 8
    wm = bench.work_model(wl, _counts(E, A, E))
    routed = 2.0 * A * 3 * d * F
    shared = 2.0 * T * 3 * d * F
    assert wm["flops_bf16"] == routed + shared
    assert round(routed / TF, 3) == 11.545 and round(shared / TF, 3) == 1.443
    assert round(wm["flops_bf16"] / TF, 3) == 12.988
    assert wm["flops_router"] == 2.0 * T * d * E                 # fp32-class, counted apart
    expert_bytes = 3 * d * F * 2                                  # 88,080,384 B of bf16 per expert
    assert expert_bytes == 88_080_384
    want = E * expert_bytes + 3 * d * F * 2 + E * d * 4 + E * 4 + 2 * T * d * 2
    assert wm["bytes"] == want and round(want / GB, 2) == 34.39
    assert wm["touched"] == E


def test_k2_prefill_up_and_down_launch_work():
    wl = get_workload("k2_prefill_t16384")
    d, F, T, E = 7168, 2048, 16384, 384
    A = T * 8
    wm = bench.work_model(wl, _counts(E, A, E))
    # up: gate and up products of the routed rows and of every token (shared)
    assert wm["up"]["flops"] == 2.0 * A * d * 2 * F + 2.0 * T * d * 2 * F
    assert round(wm["up"]["flops"] / TF, 4) == 8.6587
    up_bytes = E * 2 * F * d * 2 + 2 * F * d * 2 + T * d * 2 + A * F * 2 + T * F * 2
    assert wm["up"]["bytes"] == up_bytes
    # down: the routed rows and the shared rows, H read and Y written once
    assert wm["down"]["flops"] == 2.0 * A * F * d + 2.0 * T * F * d
    down_bytes = E * d * F * 2 + F * d * 2 + A * F * 2 + T * F * 2 + (A + T) * d * 2
    assert wm["down"]["bytes"] == down_bytes
    # combine: Y and Y_sh read, weights and positions, out written
    assert wm["combine"]["bytes"] == (A + T) * d * 2 + A * 8 + T * d * 2
    assert wm["end"] is None


def test_k2_decode_bytes_follow_the_touched_experts():
    wl = get_workload("k2_decode_t256")
    d, F, T, E = 7168, 2048, 256, 384
    A = T * 8
    for touched in (377, 200, 8):
        wm = bench.work_model(wl, _counts(E, A, touched))
        want = touched * 88_080_384 + 3 * d * F * 2 + E * d * 4 + E * 4 + 2 * T * d * 2
        assert wm["bytes"] == want and wm["touched"] == touched
    # 377 touched experts: the weight stream of one decode step
    wm = bench.work_model(wl, _counts(E, A, 377))
    assert round(wm["bytes"] / GB, 2) == 33.31
    assert round(wm["flops_bf16"] / 1e9, 1) == 202.9


def test_k3_latent_work():
    wl = get_workload("k3_latent_t4096")
    d, dl, F, T, E, K = 7168, 3584, 3072, 4096, 896, 16
    Fsh = 2 * F
    A = T * K
    wm = bench.work_model(wl, _counts(E, A, E))
    want_flops = 2.0 * A * 3 * dl * F + 2.0 * T * 3 * d * Fsh + 2.0 * T * d * dl * 2
    assert wm["flops_bf16"] == want_flops and round(want_flops / TF, 3) == 5.833
    want_bytes = (E * 3 * dl * F * 2 + 3 * d * Fsh * 2 + E * d * 4 + E * 4 + 2 * d * dl * 2
                  + 2 * T * d * 2)
    assert wm["bytes"] == want_bytes and round(want_bytes / GB, 2) == 59.70
    # the latent form's down launch holds the routed experts only; the shared
    # down projection is part of the output map [Hs | R] [Ws_down | W_lu]^T
    assert wm["down"]["flops"] == 2.0 * A * F * dl
    assert wm["end"]["flops"] == 2.0 * T * (Fsh + dl) * d


def test_fp8_weight_bytes_count_one_byte_and_the_block_scales():
    wl = get_workload("k2_decode_fp8_t256")
    d, F, E = 7168, 2048, 384
    wm = bench.work_model(wl, _counts(E, 256 * 8, E))
    per_expert = 3 * d * F + 3 * (F // 128) * (d // 128)
    assert wm["bytes"] == (E * per_expert + 3 * d * F * 2 + E * d * 4 + E * 4 + 2 * 256 * d * 2)


def test_roofline_picks_the_bound_by_intensity():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    ms = 2.0
    hot = dict(flops=ridge * 2e9 * 1.01, bytes=2e9)           # just above the ridge
    r = bench.roofline(hot, ms, "k", None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(hot["flops"] / (ms * 1e-3) / 1e12, abs=0.01)   # 2 decimals
    assert r["frac"] == pytest.approx(r["achieved"] / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    cold = dict(flops=ridge * 2e9 * 0.99, bytes=2e9)
    r = bench.roofline(cold, ms, "k", 3.0, ys=dict(hbm_read_gbs=6500.0, mfma_tflops=2100.0))
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["traffic"] == 3.0
    assert r["achieved"] == pytest.approx(2e9 / 2e-3 / 1e9, abs=0.1)             # 1000 GB/s
    assert r["frac"] == pytest.approx(1000.0 / bench.PEAK_HBM_GBS, abs=1e-4)
    assert r["frac_of_measured"] == pytest.approx(1000.0 / 6500.0, abs=1e-4)


K2_CALL = ["moe::k_split3(float const*)",
           "void moe::k_gemm_big<float, 128, 192, 2, 2, 2, 128, 0, false>(moe::GemmArgs)",
           "void moe::k_topk_gate<6>(float const*)",
           "moe::k_dispatch_masks(int const*)", "moe::k_dispatch_chunk_scan(unsigned long const*)",
           "moe::k_dispatch_scan(int)", "moe::k_dispatch_scatter(int const*)",
           "void moe::k_gemm_wide<unsigned short, 1, 1, 128, false>(moe::GemmArgs)",
           "void moe::k_gemm_wide<unsigned short, 0, 1, 128, false>(moe::GemmArgs)",
           "void moe::k_combine<unsigned short>(unsigned short const*)"]
K2_STAGES = ["split", "router", "gate", "dispatch", "dispatch", "dispatch", "dispatch", "up", "down",
             "combine"]


def test_label_stages_of_two_k2_calls():
    names = K2_CALL + K2_CALL
    got = bench.label_stages(list(enumerate(names)))
    assert [got[i] for i in range(len(names))] == K2_STAGES + K2_STAGES


def test_label_stages_of_a_latent_call():
    names = [K2_CALL[0], K2_CALL[1], "void moe::k_topk_gate<14>(float const*)"] + K2_CALL[3:7] + [
        "void moe::k_gemm_wide<unsigned short, 0, 1, 128, false>(moe::GemmArgs)",   # x_lat
        "void moe::k_gemm_wide<unsigned short, 1, 1, 128, false>(moe::GemmArgs)",   # up
        "void moe::k_gemm_wide<unsigned short, 0, 1, 128, false>(moe::GemmArgs)",   # down
        "void moe::k_combine<unsigned short>(unsigned short const*)",
        "void moe::k_gemm_wide<unsigned short, 0, 2, 128, false>(moe::GemmArgs)"]   # output map
    got = bench.label_stages(list(enumerate(names)))
    assert [got[i] for i in range(len(names))] == ["split", "router", "gate"] + ["dispatch"] * 4 + [
        "latent", "up", "down", "combine", "end"]


def test_gemm_epilogue_reads_the_template_arguments():
    assert bench.gemm_epilogue("k_gemm_wide<unsigned short, 1, 1, 128, true>") == 1
    assert bench.gemm_epilogue("k_gemm_wide<unsigned short, 0, 2, 128, false>") == 0
    assert bench.gemm_epilogue("k_gemm_big<unsigned short, 16, 512, 1, 4, 4, 64, 1, true>") == 1
    assert bench.gemm_epilogue("k_gemm_big<float, 128, 192, 2, 2, 2, 128, 0, false>") == 0
    assert bench.gemm_epilogue("k_combine<unsigned short>") is None


def test_source_hash_ignores_comments_and_layout_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "fine_grained_sparse_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = os.path.join(bench.ROOT, "fine_grained_sparse_amd", "csrc")
    for name in bench.LAYER_SOURCES:
        shutil.copy(os.path.join(src, name), csrc / name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash()
    p = csrc / "router.hip"
    text = p.read_text()
    p.write_text("// a comment\n/* and a block\n comment */\n" + text.replace("\n", "\n\n"))
    assert bench.source_hash() == h0
    p.write_text(text.replace("k_topk_gate", "k_topk_gate2", 1))
    assert bench.source_hash() != h0


def test_clock_snapshot_has_its_fields():
    import torch
    c = bench.gpu_clocks(torch)
    assert set(c) == {"sclk_mhz", "mclk_mhz", "source"}
    assert isinstance(c["source"], str) and c["source"]
    for k in ("sclk_mhz", "mclk_mhz"):
        assert c[k] is None or (isinstance(c[k], int) and c[k] > 0)
