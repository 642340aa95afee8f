"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every case prints its name before it touches the GPU.  Tolerances are
documented in tests/parity.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import fine_grained_sparse_amd as moe
import oracle
from moe_inputs import Workload, get_workload, make_layer_inputs, make_router_inputs
from parity import (RANDOM_LAYER_SEEDS, RANDOM_ROUTER_SEEDS, TIE, check_dispatch, check_output,
                    coverage_tokens, effective_routing, effective_routing_grouped, expert_weights,
                    host, log, random_layer, random_router, record_routing, weights_to_device)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _custom(**kw):
    base = dict(name="custom", T=64, d=256, E=16, K=4, F=128, n_shared=1, F_shared=128,
                d_latent=0, scale=2.827, act_dtype="bf16", w_dtype="bf16", bias_range=0.02,
                zipf_skew=False, router_only=False)
    base.update(kw)
    return Workload(**base)


def _weights(wl, dev, packed):
    w = expert_weights(dev)
    return moe.pack_weights(w, n_shared=wl.n_shared) if packed else w


def _run_forward(wl, dev, packed=False, weights=None, **kw):
    w = weights if weights is not None else _weights(wl, dev, packed)
    out, r = moe.forward(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale,
                         n_shared=wl.n_shared, return_routing=True, **kw)
    torch.cuda.synchronize()
    return out, r


def _full_parity(wl, inp, seed_note="", packed=False):
    """Run the layer on the GPU and compare every token with the oracle."""
    log(f"[gpu] forward {wl.name} T={wl.T} d={wl.d} E={wl.E} K={wl.K} "
        f"{'packed ' if packed else ''}{seed_note}")
    dev = weights_to_device(inp, DEV)
    out, r = _run_forward(wl, dev, packed)
    ref = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale, want_scores=True)
    idx_eff, w_eff, st = effective_routing(ref, r["idx"].cpu().numpy(), r["w"].cpu().numpy(),
                                           inp["b"].numpy(), wl.K, wl.scale)
    check_dispatch(r, wl.E)
    out_ref = oracle.forward_given_routing(oracle.layer_from_inputs(wl, inp), inp["x"],
                                           idx_eff, w_eff)
    case = f"{wl.name}{' packed' if packed else ''}{' ' + seed_note if seed_note else ''}"
    rec = check_output(case, out.float().cpu().numpy(), out_ref, wl.act_dtype, wl.d_latent > 0, st)
    return out, r, rec["rel_l2"]


# ---------------------------------------------------------------- router
# T = 64 and 65 sit on either side of the switch from 16-row to 128-row
# logit tiles; 1024 and 4096 split K into different numbers of planes; up to
# 32 tokens the logits are fp32 dot products (32 and 33 on either side).
@pytest.mark.parametrize("name,T", [("tiny_fp32_t128", None), ("mid_bf16_t300", None),
                                    ("k2_router_t4096", 64), ("k2_router_t4096", 65),
                                    ("k2_router_t4096", None), ("k3_latent_t4096", 1024),
                                    ("k2_router_t4096", 1), ("k2_router_t4096", 3),
                                    ("k2_router_t4096", 17), ("k2_router_t4096", 32),
                                    ("k2_router_t4096", 33), ("k3_latent_t4096", 32),
                                    ("tiny_fp32_t128", 5)])
def test_router_parity(name, T):
    wl = get_workload(name)
    log(f"[gpu] router {name} T={T or wl.T}")
    inp = make_router_inputs(wl, "cpu", seed=42, T=T)
    dev = weights_to_device(inp, DEV)
    idx, w, counts = moe.router(dev["x"], dev["W_r"], dev["b"], wl.K, wl.scale)
    torch.cuda.synchronize()
    ref = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale, want_scores=True)
    gi = idx.cpu().numpy()
    _, _, st = effective_routing(ref, gi, w.cpu().numpy(), inp["b"].numpy(), wl.K, wl.scale)
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(gi.ravel(), minlength=wl.E))
    np.testing.assert_allclose(w.double().sum(1).cpu().numpy(), float(np.float32(wl.scale)), rtol=1e-6)
    record_routing(f"router {name} T={T or wl.T}", st, T or wl.T)


def test_router_1024_experts_top16():
    wl = _custom(E=1024, K=16, d=320 - 64, T=70)
    log("[gpu] router E=1024 K=16")
    inp = make_router_inputs(wl, "cpu", seed=3)
    dev = weights_to_device(inp, DEV)
    idx, w, counts = moe.router(dev["x"], dev["W_r"], dev["b"], wl.K, wl.scale)
    torch.cuda.synchronize()
    ref = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale, want_scores=True)
    _, _, st = effective_routing(ref, idx.cpu().numpy(), w.cpu().numpy(), inp["b"].numpy(), wl.K,
                                 wl.scale)
    # the counts' LDS histogram at its largest expert count
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(idx.cpu().numpy().ravel(), minlength=wl.E))
    record_routing("router E=1024 K=16 T=70", st, wl.T)


def test_router_all_tied_and_K1():
    log("[gpu] router ties / K=1")
    T, d, E = 40, 128, 24
    x = torch.randn(T, d).to(torch.bfloat16).to(DEV)
    idx, w, _ = moe.router(x, torch.zeros(E, d, device=DEV), torch.zeros(E, device=DEV), 5)
    assert (idx.cpu() == torch.arange(5, dtype=torch.int32)).all()
    assert torch.allclose(w.cpu(), torch.full((T, 5), float(np.float32(2.827)) / 5), rtol=1e-6)
    inp = make_router_inputs(_custom(E=E, d=d, T=T), "cpu", seed=9)
    dev = weights_to_device(inp, DEV)
    idx1, w1, _ = moe.router(dev["x"], dev["W_r"], dev["b"], 1)
    assert torch.all(w1.cpu() == torch.tensor(np.float32(2.827)))


# ---------------------------------------------------------------- group-limited choice
@pytest.mark.parametrize("name,T,n_group,topk_group,bias", [
    ("tiny_fp32_t128", None, 4, 2, None),
    ("mid_bf16_t300", None, 8, 3, None),
    ("mid_bf16_t300", None, 6, 2, 0.6),        # biased scores below zero: the 0.0 fill matters
    ("k2_router_t4096", 2048, 8, 4, None),
    ("k2_router_t4096", 1024, 64, 13, None),
    ("k3_latent_t4096", 512, 8, 4, None),
])
def test_router_grouped_parity(name, T, n_group, topk_group, bias):
    wl = get_workload(name)
    log(f"[gpu] grouped router {name} T={T or wl.T} groups {n_group}/{topk_group} bias={bias}")
    r = make_router_inputs(wl, "cpu", seed=13, T=T)
    if bias is not None:
        g = torch.Generator().manual_seed(17)
        r["b"] = (torch.rand(wl.E, generator=g) * 2 - 1) * bias - 0.45
    ref = oracle.router_grouped(r["x"], r["W_r"], r["b"], wl.K, wl.scale, n_group, topk_group,
                                want_scores=True)
    dev = weights_to_device(r, DEV)
    idx, w, counts = moe.router(dev["x"], dev["W_r"], dev["b"], wl.K, wl.scale,
                                n_group=n_group, topk_group=topk_group)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    _, _, st = effective_routing_grouped(ref, gi, w.cpu().numpy(), wl.K, wl.scale)
    assert np.array_equal(np.bincount(gi.ravel(), minlength=wl.E), counts.cpu().numpy())
    if bias is not None:  # the case is exercised: many biased scores are below the 0.0 fill
        v = ref["scores"] + r["b"].double().numpy()[None, :]
        assert (v < 0).mean() > 0.2
    record_routing(f"grouped router {name} T={T or wl.T} {n_group}/{topk_group}"
                   f"{' neg-bias' if bias is not None else ''}", st, T or wl.T)
    assert st["near_tie"] <= max(3, (T or wl.T) // 100)


@pytest.mark.parametrize("seed", list(RANDOM_ROUTER_SEEDS))
def test_router_random_shapes(seed):
    # Seeded random router shapes within the ABI's limits (random_router in
    # tests/parity.py), with and without the group-limited choice.
    kw, n_group, topk_group = random_router(seed)
    wl = Workload(**kw)
    log(f"[gpu] router {wl.name} T={wl.T} d={wl.d} E={wl.E} K={wl.K} {wl.act_dtype} "
        f"groups {n_group}/{topk_group}")
    r = make_router_inputs(wl, "cpu", seed=200 + seed)
    dev = weights_to_device(r, DEV)
    idx, w, counts = moe.router(dev["x"], dev["W_r"], dev["b"], wl.K, wl.scale, n_group=n_group,
                                topk_group=topk_group)
    torch.cuda.synchronize()
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    if n_group > 1:
        ref = oracle.router_grouped(r["x"], r["W_r"], r["b"], wl.K, wl.scale, n_group, topk_group,
                                    want_scores=True)
        _, _, st = effective_routing_grouped(ref, gi, gw, wl.K, wl.scale)
    else:
        ref = oracle.router(r["x"], r["W_r"], r["b"], wl.K, wl.scale, want_scores=True)
        _, _, st = effective_routing(ref, gi, gw, r["b"].numpy(), wl.K, wl.scale)
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(gi.ravel(), minlength=wl.E))
    np.testing.assert_allclose(gw.astype(np.float64).sum(1), float(np.float32(wl.scale)), rtol=1e-6)
    record_routing(f"{wl.name} T={wl.T} E={wl.E} K={wl.K} d={wl.d} {wl.act_dtype} "
                   f"{n_group}/{topk_group}", st, wl.T)


def test_forward_with_grouped_routing():
    wl = get_workload("mid_bf16_t300")
    log("[gpu] forward mid_bf16_t300 with 8 groups / 3 kept")
    inp = make_layer_inputs(wl, "cpu", seed=42)
    dev = weights_to_device(inp, DEV)
    out, r = moe.forward(dev["x"], dev["W_r"], dev["b"], expert_weights(dev), wl.K, wl.scale,
                         n_shared=wl.n_shared, return_routing=True, n_group=8, topk_group=3)
    torch.cuda.synchronize()
    ref = oracle.router_grouped(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale, 8, 3,
                                want_scores=True)
    idx_eff, w_eff, st = effective_routing_grouped(ref, r["idx"].cpu().numpy(),
                                                   r["w"].cpu().numpy(), wl.K, wl.scale)
    check_dispatch(r, wl.E)
    out_ref = oracle.forward_given_routing(oracle.layer_from_inputs(wl, inp), inp["x"], idx_eff, w_eff)
    check_output("mid_bf16_t300 grouped 8/3", out.float().cpu().numpy(), out_ref, wl.act_dtype,
                 False, st)


# ---------------------------------------------------------------- expert-parallel slices
def _slice_weights(w, e0, e1, shared):
    """The weights one GPU holds for experts e0 .. e1 - 1 (plus the shared
    experts if it runs them; the latent maps always)."""
    s = {k: w[k][e0:e1].contiguous() for k in ("W_gate", "W_up", "W_down")}
    for k in ("W_gate_scale", "W_up_scale", "W_down_scale"):
        if w.get(k) is not None:
            s[k] = w[k][e0:e1].contiguous()
    for k in ("W_lat_down", "W_lat_up") + (("Ws_gate", "Ws_up", "Ws_down") if shared else ()):
        if w.get(k) is not None:
            s[k] = w[k]
    return s


def _slice_reference(wl, inp, gi, gw, e0, e1, shared):
    """The oracle layer with the other slices' gate weights set to zero
    (their ids moved inside the slice, so any id is a valid index)."""
    local = (gi >= e0) & (gi < e1)
    wl_s = dataclasses.replace(wl, n_shared=wl.n_shared if shared else 0,
                               F_shared=wl.F_shared if shared else 0)
    return oracle.forward_given_routing(oracle.layer_from_inputs(wl_s, inp), inp["x"],
                                        np.where(local, gi, e0), np.where(local, gw, 0.0)), local


@pytest.mark.parametrize("name,packed", [("mid_bf16_t300", False), ("mid_bf16_t300", True),
                                         ("mid_fp8_t300", True), ("mid_latent_t200", True),
                                         ("mid_fp8_latent_t200", True), ("mid_fp32_t77", False)])
def test_forward_slice_parity(name, packed):
    # Expert-parallel slices under the layer's GPU routing: one expert (with
    # the shared experts), fewer experts than K, then two halves of the
    # rest; every token against the oracle.
    wl = get_workload(name)
    inp = make_layer_inputs(wl, "cpu", seed=21)
    dev = weights_to_device(inp, DEV)
    idx, w, _ = moe.router(dev["x"], dev["W_r"], dev["b"], wl.K, wl.scale)
    torch.cuda.synchronize()
    gi, gw = idx.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    full = expert_weights(dev)
    E, k1 = wl.E, max(2, wl.K - 1)
    for i, (e0, e1) in enumerate([(0, 1), (1, k1), (k1, E // 2), (E // 2, E)]):
        shared = i == 0 and wl.n_shared > 0
        sw = _slice_weights(full, e0, e1, shared)
        if packed:
            sw = moe.pack_weights(sw, n_shared=wl.n_shared if shared else None)
        log(f"[gpu] slice {name} experts {e0}..{e1 - 1} of {E}{' + shared' if shared else ''}"
            f"{' packed' if packed else ''}")
        out, disp = moe.forward_slice(dev["x"], idx, w, sw, e0, E,
                                      n_shared=wl.n_shared if shared else None, return_dispatch=True)
        torch.cuda.synchronize()
        ref, local = _slice_reference(wl, inp, gi, gw, e0, e1, shared)
        counts = np.bincount(gi[local] - e0, minlength=e1 - e0)
        assert np.array_equal(disp["counts"].cpu().numpy(), counts)
        assert np.array_equal(disp["offsets"].cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))
        check_output(f"{name}{' packed' if packed else ''} slice {e0}..{e1 - 1}"
                     f"{' + shared' if shared else ''}", out.float().cpu().numpy(), ref, wl.act_dtype,
                     wl.d_latent > 0)


@pytest.mark.parametrize("seed", list(range(24)))
def test_forward_slice_random_layers(seed):
    # a random slice of each seeded random layer (all modes, both tile
    # sizes), with the shared experts in every other one, under the
    # layer's GPU routing: every token against the oracle
    kw, packed, hot = random_layer(seed)
    wl = Workload(**kw)
    rng = np.random.default_rng(500 + seed)
    e0 = int(rng.integers(0, wl.E))
    e1 = int(rng.integers(e0 + 1, wl.E + 1))
    shared = wl.n_shared > 0 and seed % 2 == 0
    log(f"[gpu] slice {wl.name} T={wl.T} E={wl.E} K={wl.K}: experts {e0}..{e1 - 1}"
        f"{' + shared' if shared else ''}")
    inp = make_layer_inputs(wl, "cpu", seed=100 + seed)
    if hot is not None:
        inp["b"][hot] = 10.0
    dev = weights_to_device(inp, DEV)
    idx, w, _ = moe.router(dev["x"], dev["W_r"], dev["b"], wl.K, wl.scale)
    torch.cuda.synchronize()
    sw = _slice_weights(expert_weights(dev), e0, e1, shared)
    if packed:
        sw = moe.pack_weights(sw, n_shared=wl.n_shared if shared else None)
    out = moe.forward_slice(dev["x"], idx, w, sw, e0, wl.E, n_shared=wl.n_shared if shared else None)
    torch.cuda.synchronize()
    ref, _ = _slice_reference(wl, inp, idx.cpu().numpy(), w.cpu().numpy().astype(np.float64), e0, e1,
                              shared)
    check_output(f"{wl.name} slice {e0}..{e1 - 1}{' + shared' if shared else ''}",
                 out.float().cpu().numpy(), ref, wl.act_dtype, wl.d_latent > 0)


@pytest.mark.parametrize("name,packed", [("mid_bf16_t300", True), ("mid_fp8_t300", True),
                                         ("mid_latent_t200", False), ("tiny_fp32_t128", False)])
def test_forward_slice_whole_range_is_forward(name, packed):
    # all experts and the shared ones, under moe_forward's own routing: the
    # same kernels in the same order, so the same bits
    wl = get_workload(name)
    log(f"[gpu] slice {name}: whole range against moe_forward")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=22), DEV)
    w = expert_weights(dev)
    if packed:
        w = moe.pack_weights(w, n_shared=wl.n_shared)
    ref, r = moe.forward(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=wl.n_shared,
                         return_routing=True)
    out, disp = moe.forward_slice(dev["x"], r["idx"], r["w"], w, 0, wl.E, n_shared=wl.n_shared,
                                  return_dispatch=True)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if ref.dtype == torch.bfloat16 else (lambda t: t)
    assert torch.equal(bits(out), bits(ref))
    for k in ("counts", "offsets"):
        assert torch.equal(disp[k], r[k])
    n = wl.T * wl.K
    assert torch.equal(disp["sorted_token"][:n], r["sorted_token"][:n])


def test_forward_slices_sum_to_the_layer():
    # fp32 layer split over four GPUs (8 experts each, the first with the
    # shared expert): the partial outputs add up to the layer
    wl = get_workload("tiny_fp32_t128")
    log("[gpu] slices of tiny_fp32_t128 summed against moe_forward")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=23), DEV)
    w = expert_weights(dev)
    ref, r = moe.forward(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=wl.n_shared,
                         return_routing=True)
    total = torch.zeros_like(ref, dtype=torch.float64)
    for g in range(4):
        e0, e1 = 8 * g, 8 * g + 8
        total += moe.forward_slice(dev["x"], r["idx"], r["w"], _slice_weights(w, e0, e1, g == 0), e0,
                                   wl.E, n_shared=wl.n_shared if g == 0 else None).double()
    torch.cuda.synchronize()
    err = float((total - ref.double()).norm() / ref.double().norm())
    log(f"  sum of 4 slices vs layer: relative L2 {err:.2e}")
    assert err < 1e-6


@pytest.mark.parametrize("n_shared", [0, 1])
def test_forward_slice_skips_ids_outside_it(n_shared):
    # routing ids anywhere in [-40, 60) for a slice of experts 4 .. 7 of 16:
    # only those four count; a token with none of them gets the shared
    # experts' output, or zeros
    wl = _custom(E=16, K=4, T=150, n_shared=n_shared, F_shared=128 if n_shared else 0)
    log(f"[gpu] slice 4..7 of 16 under ids in [-40, 60), n_shared={n_shared}")
    inp = make_layer_inputs(wl, "cpu", seed=24)
    g = torch.Generator().manual_seed(25)
    gi = torch.stack([torch.randperm(100, generator=g)[:wl.K] - 40 for _ in range(wl.T)]).to(torch.int32)
    gw = torch.rand(wl.T, wl.K, generator=g)
    gi[:10] = torch.tensor([-1, 8, 16, 59], dtype=torch.int32)   # no expert of the slice
    dev = weights_to_device(inp, DEV)
    sw = _slice_weights(expert_weights(dev), 4, 8, n_shared > 0)
    out = moe.forward_slice(dev["x"], gi.to(DEV), gw.to(DEV), sw, 4, 16,
                            n_shared=n_shared or None)
    torch.cuda.synchronize()
    ref, local = _slice_reference(wl, inp, gi.numpy(), gw.numpy().astype(np.float64), 4, 8, n_shared > 0)
    assert not local[:10].any() and local.any()
    if n_shared == 0:
        assert bool((out[:10] == 0).all())
    check_output(f"slice 4..7 of 16, ids in [-40, 60), shared {n_shared}", out.float().cpu().numpy(), ref,
                 wl.act_dtype, False)


# ---------------------------------------------------------------- bias update
@pytest.mark.parametrize("E", [1, 7, 384, 896, 1024])
def test_bias_update_parity(E):
    log(f"[gpu] bias update E={E}")
    g = torch.Generator().manual_seed(E)
    counts = torch.randint(0, 50, (E,), generator=g, dtype=torch.int32)
    if E >= 7:
        counts[:3] = int(counts.float().mean().round())   # some near the mean
        counts[3] = 0
    b = (torch.rand(E, generator=g) - 0.5) * 0.1
    ref = oracle.bias_update(counts.numpy(), b.numpy(), gamma=1e-3)
    bd = b.to(DEV)
    moe.bias_update(counts.to(DEV), bd, 1e-3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bd.cpu().numpy(), ref)   # bit for bit


def test_bias_update_from_the_layers_own_counts():
    # the counts moe_forward returns feed the update directly
    wl = get_workload("mid_bf16_t300")
    log("[gpu] bias update from moe_forward counts")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=42), DEV)
    _, r = _run_forward(wl, dev)
    b0 = dev["b"].clone()
    moe.bias_update(r["counts"], dev["b"], 1e-3)
    torch.cuda.synchronize()
    ref = oracle.bias_update(r["counts"].cpu().numpy(), b0.cpu().numpy())
    np.testing.assert_array_equal(dev["b"].cpu().numpy(), ref)


@pytest.mark.parametrize("name,T", [("tiny_fp32_t128", None), ("mid_bf16_t300", None),
                                    ("k3_latent_t4096", None), ("k2_router_t4096", 16384),
                                    ("k3_latent_t4096", 24)])
def test_bias_quantile_parity(name, T):
    wl = get_workload(name)
    T = T or wl.T
    log(f"[gpu] quantile bias {name} T={T}")
    r = make_router_inputs(wl, "cpu", seed=29, T=T)
    b_ref, th_ref = oracle.bias_quantile(r["x"], r["W_r"], wl.K)
    dev = weights_to_device(r, DEV)
    b = moe.bias_quantile(dev["x"], dev["W_r"], wl.K)
    torch.cuda.synchronize()
    # fp32 scores against fp64 ones: each threshold is an order statistic of
    # scores within ~1e-6 of the oracle's, the mean adds no more
    err = np.abs(b.cpu().numpy().astype(np.float64) - b_ref).max()
    log(f"  max |b - b_ref| = {err:.2e}")
    assert err <= 1e-5


# ---------------------------------------------------------------- whole layer, every token
@pytest.mark.parametrize("name,packed", [("tiny_fp32_t128", False), ("mid_fp32_t77", False),
                                         ("mid_bf16_t300", False), ("mid_latent_t200", False),
                                         ("mid_bf16_t300", True), ("mid_latent_t200", True),
                                         ("mid_fp8_t300", True), ("mid_fp8_latent_t200", True)])
def test_forward_parity_every_token(name, packed):
    wl = get_workload(name)
    _full_parity(wl, make_layer_inputs(wl, "cpu", seed=42), packed=packed)


@pytest.mark.parametrize("packed", [False, True], ids=["rows", "packed"])
@pytest.mark.parametrize("case", ["one_token", "K_equals_E", "no_shared", "skewed_few_experts",
                                  "latent_no_shared", "large_tiles", "large_tiles_latent",
                                  "half_tiles", "max_limits", "prefill_k8", "prefill_k6_two_shared",
                                  "prefill_k16", "decode_hot_expert", "narrow_hot_expert"])
def test_forward_edge_cases(case, packed):
    if case == "one_token":
        wl = _custom(T=1)
    elif case == "K_equals_E":
        wl = _custom(E=16, K=16, T=33)
    elif case == "no_shared":
        wl = _custom(n_shared=0, F_shared=0, T=130)
    elif case == "skewed_few_experts":
        wl = _custom(E=40, K=3, T=200)
    elif case == "latent_no_shared":
        wl = _custom(d_latent=128, n_shared=0, F_shared=0, T=90, scale=1.0)
    elif case == "large_tiles":  # enough rows per expert for the 128-row tiles, ragged tails
        wl = _custom(E=6, K=2, T=700, d=384, F=192, n_shared=2, F_shared=64)
    elif case == "large_tiles_latent":  # 128-row tiles for the experts and the dense
        # latent maps (T >= 512), two K segments in the last GEMM, N tails inside a
        # 512-wide tile
        wl = _custom(E=5, K=2, T=1100, d=320, F=192, n_shared=1, F_shared=128, d_latent=192,
                     scale=1.0)
    elif case == "prefill_k8":  # prefill-sized: 128-row expert tiles and 128-row dense tiles
        # (T >= 512), a ragged last row tile
        wl = _custom(E=32, K=8, T=1100, d=256, F=128, n_shared=1, F_shared=128)
    elif case == "prefill_k6_two_shared":  # N tail (d = 320 in 512-column tiles), two shared
        wl = _custom(E=24, K=6, T=1030, d=320, F=128, n_shared=2, F_shared=64)
    elif case == "prefill_k16":
        wl = _custom(E=64, K=16, T=1024, d=192, F=64, n_shared=1, F_shared=64)
    elif case == "max_limits":  # the ABI's limits: 1024 experts, top-16, 8 shared experts,
        # the narrowest widths (64)
        wl = _custom(E=1024, K=16, T=300, d=192, F=64, n_shared=8, F_shared=64)
    elif case == "decode_hot_expert":  # 6.25 rows per expert on average (16-row tiles,
        # below the switch at 10), but expert 0 takes all 200 tokens: 13 tiles of it;
        # 512-wide tiles (154 workgroups or more)
        wl = _custom(E=64, K=2, T=200, d=1024, F=512, F_shared=512)
    elif case == "narrow_hot_expert":  # the same routing at d = 256, F = 128: the
        # 512-wide tiles would make 77 workgroups, so the 16 x 256 ones serve it
        wl = _custom(E=64, K=2, T=200)
    else:  # half_tiles: expert 0 gets four full 128-row tiles + 8 rows, the others ~35
        # rows each: 128-row tiles that are mostly padding
        wl = _custom(E=16, K=2, T=520, d=256, F=128, n_shared=1, F_shared=128)
    inp = make_layer_inputs(wl, "cpu", seed=5)
    if case == "skewed_few_experts":
        inp["b"][:3] = 10.0     # every token picks experts 0, 1, 2; the rest get none
    if case in ("half_tiles", "decode_hot_expert", "narrow_hot_expert"):
        inp["b"][0] = 10.0
    _, r, _ = _full_parity(wl, inp, case, packed=packed)
    if case in ("decode_hot_expert", "narrow_hot_expert"):
        assert r["counts"].cpu().numpy()[0] == 200 and wl.T * wl.K < 10 * wl.E
    if case == "skewed_few_experts":
        c = r["counts"].cpu().numpy()
        assert c[:3].tolist() == [200, 200, 200] and c[3:].sum() == 0
    if case == "half_tiles":
        c = r["counts"].cpu().numpy()
        assert c[0] == 520 and 0 < c[1:].max() <= 64


@pytest.mark.parametrize("case", ["one_token", "K_equals_E", "no_shared", "latent_no_shared",
                                  "large_tiles", "large_tiles_latent", "half_tiles", "prefill_k8",
                                  "decode_hot_expert", "decode_ragged_n"])
def test_forward_fp8_edge_cases(case):
    # FP8 routed experts (packed): 16-row tiles below 10 rows per expert on
    # average, 128-row tiles above; the shared experts ride in the same
    # launches as a bf16 group, the latent maps run as bf16 launches of
    # their own.  Block-scale rows past N (down projections narrower than
    # the tile's weight rows) are clamped.
    fp8 = dict(w_dtype="fp8")
    if case == "one_token":
        wl = _custom(T=1, **fp8)
    elif case == "K_equals_E":
        wl = _custom(E=16, K=16, T=33, **fp8)
    elif case == "no_shared":
        wl = _custom(n_shared=0, F_shared=0, T=130, **fp8)
    elif case == "latent_no_shared":
        wl = _custom(d=320, d_latent=128, n_shared=0, F_shared=0, T=90, scale=1.0, **fp8)
    elif case == "large_tiles":
        wl = _custom(E=6, K=2, T=700, d=384, F=256, n_shared=2, F_shared=64, **fp8)
    elif case == "large_tiles_latent":  # 128-row expert tiles; bf16 128-row dense tiles
        wl = _custom(E=5, K=2, T=1100, d=320, F=256, n_shared=1, F_shared=128, d_latent=256,
                     scale=1.0, **fp8)
    elif case == "prefill_k8":  # prefill-sized tiles, top-8
        wl = _custom(E=32, K=8, T=1100, d=256, F=128, n_shared=1, F_shared=128, **fp8)
    elif case == "decode_hot_expert":  # 16-row tiles, expert 0 in 13 of them
        wl = _custom(E=64, K=2, T=200, **fp8)
    elif case == "decode_ragged_n":  # 16-row tiles (256 weight rows, 128 SwiGLU columns):
        # up F = 384 in three N tiles, down d = 640 in two and a half,
        # the shared expert's F = 192 in one and a half
        wl = _custom(E=32, K=2, T=100, d=640, F=384, F_shared=192, **fp8)
    else:  # half_tiles: expert 0 takes every token, the others ~35 rows each
        wl = _custom(E=16, K=2, T=520, **fp8)
    inp = make_layer_inputs(wl, "cpu", seed=6)
    if case in ("half_tiles", "decode_hot_expert"):
        inp["b"][0] = 10.0
    _full_parity(wl, inp, "fp8 " + case, packed=True)


@pytest.mark.parametrize("seed", list(RANDOM_LAYER_SEEDS))
def test_forward_random_layers(seed):
    # Seeded random layers within the ABI's limits (random_layer in
    # tests/parity.py): every token against the oracle, whichever tiles the
    # planner picks for the drawn shape and batch.
    kw, packed, hot = random_layer(seed)
    wl = Workload(**kw)
    inp = make_layer_inputs(wl, "cpu", seed=100 + seed)
    if hot is not None:
        inp["b"][hot] = 10.0  # every token selects it
    note = (f"F={wl.F} shared={wl.n_shared}x{wl.F_shared} d_latent={wl.d_latent} "
            f"{wl.act_dtype}/{wl.w_dtype}" + (f" hot={hot}" if hot is not None else ""))
    _, r, _ = _full_parity(wl, inp, note, packed=packed)
    if hot is not None:
        assert r["counts"].cpu().numpy()[hot] == wl.T


@pytest.mark.parametrize("tiles", ["16-row", "128-row"])
@pytest.mark.parametrize("exps", [(0, 1, 2), (198, 199, 200)])
def test_forward_fp8_extreme_block_scales(tiles, exps):
    # E8M0 exponents at both ends of the range on every down projection
    # block: 2^-127 .. 2^-125 (exponent 0 is the smallest scale, not zero)
    # and 2^71 .. 2^73.  Without a shared expert the layer output is the
    # routed sum alone, so it scales with them and the per-token check
    # sees a scale decoded wrong.  The down codes are kept at magnitude 8
    # or more, so every scaled weight stays in bf16's normal range (the
    # range the library's FP8 contract covers).  The gate and up
    # projections keep their generated scales.
    T = 40 if tiles == "16-row" else 600
    wl = _custom(E=8, K=2, T=T, n_shared=0, F_shared=0, w_dtype="fp8")
    inp = make_layer_inputs(wl, "cpu", seed=9)
    g = torch.Generator().manual_seed(9)
    pick = torch.randint(0, 3, inp["W_down_scale"].shape, generator=g)
    inp["W_down_scale"] = torch.tensor(exps, dtype=torch.uint8)[pick]
    c = inp["W_down"].float()
    c = torch.where(c.abs() < 8, torch.where(c < 0, -8.0, 8.0), c)
    inp["W_down"] = c.to(torch.float8_e4m3fn)
    _, _, rel = _full_parity(wl, inp, f"fp8 down scales 2^({exps[0]}-127).. {tiles}", packed=True)
    assert rel < 2e-2


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_forward_tile_row_buckets(w_dtype):
    # Experts with 1, 15, 16, 17, ... 129, 200 rows: the ragged last 128-row
    # tile of each expert runs the 32-, 64-, 96- or 128-row body; every
    # bucket edge appears, and every 16-row MFMA block edge inside a body.
    # Token t is steered to expert f(t) by a one-hot feature that only
    # W_r[f(t)] weights heavily (K = 1, wide margins).
    sizes = [1] + [16 * m + o for m in range(1, 9) for o in (-1, 0, 1)] + [200]
    E, T, d = len(sizes), sum(sizes), 256
    assert T >= 64 * E  # the 128-row register-fed tiles serve this layer
    wl = _custom(E=E, K=1, T=T, d=d, F=128, w_dtype=w_dtype)
    inp = make_layer_inputs(wl, "cpu", seed=8)
    g = torch.Generator().manual_seed(8)
    owner = torch.cat([torch.full((c,), e, dtype=torch.int64) for e, c in enumerate(sizes)])
    owner = owner[torch.randperm(T, generator=g)]
    x = torch.randn((T, d), generator=g) * 0.1
    x[torch.arange(T), owner] += 4.0
    inp["x"] = x.to(torch.bfloat16)
    W_r = torch.randn((E, d), generator=g) * 0.01
    W_r[torch.arange(E), torch.arange(E)] = 8.0
    inp["W_r"], inp["b"] = W_r.contiguous(), torch.zeros(E)
    _, r, _ = _full_parity(wl, inp, f"{w_dtype} row buckets", packed=True)
    assert r["counts"].cpu().tolist() == sizes


def test_forward_many_tiles_per_expert():
    # Experts averaging more than 128 rows: one to four 128-row tiles per
    # expert, last tiles on both sides of every 32-row body edge, and N
    # tails in both projections (F = 192: the up projection's 256-column
    # tile is three-quarters full; d = 320: the down projection's
    # 512-column tile holds 320).
    sizes = [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 159, 160, 161, 191, 192, 193, 300, 384,
             385, 500]
    E, T, d = len(sizes), sum(sizes), 320
    assert T >= 128 * E
    wl = _custom(E=E, K=1, T=T, d=d, F=192, n_shared=1, F_shared=128)
    inp = make_layer_inputs(wl, "cpu", seed=9)
    g = torch.Generator().manual_seed(9)
    owner = torch.cat([torch.full((c,), e, dtype=torch.int64) for e, c in enumerate(sizes)])
    owner = owner[torch.randperm(T, generator=g)]
    x = torch.randn((T, d), generator=g) * 0.1
    x[torch.arange(T), owner] += 4.0
    inp["x"] = x.to(torch.bfloat16)
    W_r = torch.randn((E, d), generator=g) * 0.01
    W_r[torch.arange(E), torch.arange(E)] = 8.0
    inp["W_r"], inp["b"] = W_r.contiguous(), torch.zeros(E)
    _, r, _ = _full_parity(wl, inp, "many tiles per expert", packed=True)
    assert r["counts"].cpu().tolist() == sizes


def test_forward_zero_tokens():
    wl = _custom(T=0)
    log("[gpu] forward T=0")
    inp = make_layer_inputs(wl, "cpu", seed=1)
    dev = weights_to_device(inp, DEV)
    out, r = _run_forward(wl, dev)
    assert out.shape == (0, wl.d)
    assert r["counts"].cpu().sum() == 0 and r["offsets"].cpu().sum() == 0


def test_forward_deterministic_and_independent_of_workspace_contents():
    wl = get_workload("mid_bf16_t300")
    log("[gpu] determinism mid_bf16_t300")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=42), DEV)
    ws = moe.Workspace()
    D = moe.desc(T=wl.T, d=wl.d, E=wl.E, K=wl.K, F=wl.F, n_shared=wl.n_shared,
                 F_shared=wl.F_shared, scale=wl.scale)
    buf = ws.get(torch.device(DEV), moe.workspace_size(D, True))
    buf.fill_(0)
    out1, r1 = _run_forward(wl, dev, workspace=ws)
    buf.fill_(0xFF)             # NaN patterns everywhere in the scratch
    out2, r2 = _run_forward(wl, dev, workspace=ws)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k


def test_forward_on_a_side_stream_and_replayed_from_a_graph():
    # The layer only enqueues kernels on the stream it is given: the same
    # call on a second stream, and a HIP graph captured from it and replayed
    # with eager work in between, give the default stream's bits.
    wl = get_workload("mid_bf16_t300")
    log("[gpu] side stream and graph replay mid_bf16_t300")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=42), DEV)
    w = _weights(wl, dev, packed=True)
    ref, _ = _run_forward(wl, dev, weights=w)
    ws = moe.Workspace()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):  # the second call also runs on a warm workspace
            moe.forward(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=wl.n_shared,
                        out=out, workspace=ws, stream=side)
    side.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        moe.forward(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=wl.n_shared,
                    out=out, workspace=ws, stream=side)
    for rep in range(3):
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"


def test_two_streams_get_separate_default_workspaces():
    # Two calls in flight on two streams with the default workspace: each
    # stream gets scratch of its own, so both give the default stream's bits.
    wl = get_workload("mid_bf16_t300")
    log("[gpu] two streams, default workspace, mid_bf16_t300")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=42), DEV)
    w = _weights(wl, dev, packed=True)
    ref, _ = _run_forward(wl, dev, weights=w)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for s in streams:
            outs.append(moe.forward(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale,
                                    n_shared=wl.n_shared, stream=s))
    for s in streams:
        s.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    keys = {k for k in moe._default_ws._buf if k[1] in {s.cuda_stream for s in streams}}
    assert len(keys) == 2


# ---------------------------------------------------------------- full sizes
# Decode batches (256 tokens): every token.  Prefill and K3 batches: a
# sample that puts a checked row in every M tile of every expert (and in
# every expert's ragged last tile) and in every shared-expert tile, plus
# random tokens (512 of the K2 prefill batch, 256 of the K3 batch), the
# near-tie tokens, the hottest and coldest experts' tokens and the last
# token.
@pytest.mark.parametrize("name,packed", [(n, p) for n in ("k2_decode_t256", "k2_prefill_t16384",
                                                            "k3_latent_t4096") for p in (False, True)]
                         + [("k2_decode_fp8_t256", True), ("k2_prefill_fp8_t16384", True)])
def test_forward_parity_full_size(name, packed):
    wl = get_workload(name)
    log(f"[gpu] full-size {name}: generating inputs on the GPU")
    inp = make_layer_inputs(wl, DEV, seed=42)
    w = None
    if packed:
        log(f"[gpu] full-size {name}: packing the weights")
        w = moe.pack_weights(expert_weights(inp), n_shared=wl.n_shared)
    log(f"[gpu] full-size {name}: moe_forward ({'packed' if packed else 'row-major'} weights)")
    out, r = _run_forward(wl, inp, weights=w)
    del w
    x_h, Wr_h, b_h = host(inp["x"]), host(inp["W_r"]), host(inp["b"])
    log(f"[cpu] oracle router over all {wl.T} tokens")
    ref = oracle.router(x_h, Wr_h, b_h, wl.K, wl.scale, want_scores=True)
    idx_eff, w_eff, st = effective_routing(ref, r["idx"].cpu().numpy(), r["w"].cpu().numpy(),
                                           b_h.numpy(), wl.K, wl.scale)
    check_dispatch(r, wl.E)
    counts = r["counts"].cpu().numpy()
    if wl.T <= 256:
        toks = np.arange(wl.T)
    else:
        toks = coverage_tokens(wl.T, wl.K, counts, r["offsets"].cpu().numpy(),
                               r["sorted_token"].cpu().numpy(), idx_eff, ref["gap"], bm=128,
                               n_random=512 if wl.T >= 16384 else 256)
    experts = set(idx_eff[toks].ravel().tolist())
    log(f"[cpu] copying {len(experts)} experts to the host; oracle over {len(toks)} tokens")
    names = ("W_gate", "W_up", "W_down") + (("W_gate_scale", "W_up_scale", "W_down_scale")
                                              if wl.w_dtype == "fp8" else ())
    per = {k: [host(inp[k][e]) if e in experts else None for e in range(wl.E)] for k in names}
    lay = oracle.Layer(d=wl.d, E=wl.E, K=wl.K, F=wl.F, scale=wl.scale, W_r=Wr_h, b=b_h,
                       W_gate=per["W_gate"], W_up=per["W_up"], W_down=per["W_down"],
                       W_gate_scale=per.get("W_gate_scale"), W_up_scale=per.get("W_up_scale"),
                       W_down_scale=per.get("W_down_scale"),
                       n_shared=wl.n_shared, F_shared=wl.F_shared,
                       Ws_gate=host(inp["Ws_gate"]), Ws_up=host(inp["Ws_up"]),
                       Ws_down=host(inp["Ws_down"]), d_latent=wl.d_latent,
                       W_lat_down=host(inp["W_lat_down"]) if wl.d_latent else None,
                       W_lat_up=host(inp["W_lat_up"]) if wl.d_latent else None)
    out_ref = oracle.forward_given_routing(lay, x_h[toks], idx_eff[toks], w_eff[toks])
    got = out[torch.from_numpy(toks).to(DEV)].float().cpu().numpy()
    del inp, out, r, per, lay
    torch.cuda.empty_cache()
    hist = f"{counts.min()}/{counts.mean():.1f}/{counts.max()}"
    check_output(f"{name}{' packed' if packed else ''}", got, out_ref, wl.act_dtype,
                 wl.d_latent > 0, st, extra=dict(hist=hist, experts=len(experts)))


@pytest.mark.parametrize("packed,w_dtype", [(False, "bf16"), (True, "bf16"), (True, "fp8")])
def test_forward_past_32bit_offsets(packed, w_dtype):
    # x [300000, 8192] (2.46e9 elements, 4.9 GB) and the routed outputs
    # [600000, 8192] (9.8 GB): element offsets past 2^31 and byte offsets
    # past 2^32 in the row gathers, the stores and the combine.  Sampled
    # tokens cover every M tile of every expert (the rows past the 32-bit
    # limits included) plus 256 random ones.
    wl = _custom(T=300000, d=8192, E=16, K=2, F=128, n_shared=1, F_shared=128, w_dtype=w_dtype)
    tag = f"{'packed ' if packed else ''}{w_dtype}"
    log(f"[gpu] past 32-bit offsets ({tag}): generating inputs on the GPU")
    inp = make_layer_inputs(wl, DEV, seed=21)
    w = moe.pack_weights(expert_weights(inp), n_shared=wl.n_shared) if packed else None
    log(f"[gpu] past 32-bit offsets ({tag}): moe_forward")
    out, r = _run_forward(wl, inp, weights=w)
    del w
    x_h, Wr_h, b_h = host(inp["x"]), host(inp["W_r"]), host(inp["b"])
    log(f"[cpu] oracle router over all {wl.T} tokens")
    ref = oracle.router(x_h, Wr_h, b_h, wl.K, wl.scale, want_scores=True)
    idx_eff, w_eff, st = effective_routing(ref, r["idx"].cpu().numpy(), r["w"].cpu().numpy(),
                                           b_h.numpy(), wl.K, wl.scale)
    check_dispatch(r, wl.E)
    toks = coverage_tokens(wl.T, wl.K, r["counts"].cpu().numpy(), r["offsets"].cpu().numpy(),
                           r["sorted_token"].cpu().numpy(), idx_eff, ref["gap"], bm=128, n_random=256)
    assert toks.max() >= 2 ** 31 // wl.d  # rows whose x elements lie past 2^31
    log(f"[cpu] oracle over {len(toks)} tokens")
    lay = oracle.layer_from_inputs(wl, {k: host(v) if isinstance(v, torch.Tensor) else v
                                        for k, v in inp.items() if k != "x"})
    out_ref = oracle.forward_given_routing(lay, x_h[toks], idx_eff[toks], w_eff[toks])
    got = out[torch.from_numpy(toks).to(DEV)].float().cpu().numpy()
    del inp, out, r, lay
    torch.cuda.empty_cache()
    check_output(f"past 32-bit offsets {tag}", got, out_ref, wl.act_dtype, False, st,
                 extra=dict(tokens=len(toks)))


def test_nan_rows_still_route_to_valid_experts():
    # Unsupported input, but it must not produce invalid expert ids: a NaN
    # score ranks below every number, so each token still selects K
    # distinct experts in range and the layer runs to completion.
    wl = _custom(E=40, K=5, T=96)
    log("[gpu] NaN rows")
    inp = make_layer_inputs(wl, "cpu", seed=23)
    inp["x"][::7] = float("nan")
    dev = weights_to_device(inp, DEV)
    idx, w, counts = moe.router(dev["x"], dev["W_r"], dev["b"], wl.K, wl.scale)
    out, r = _run_forward(wl, dev)
    gi = idx.cpu().numpy()
    assert gi.min() >= 0 and gi.max() < wl.E
    assert np.all(np.diff(gi, axis=1) > 0)
    assert int(counts.cpu().sum()) == wl.T * wl.K
    assert np.array_equal(r["idx"].cpu().numpy(), gi)
    check_dispatch(r, wl.E)
    ok = np.isfinite(inp["x"].float().numpy()).all(1)
    assert torch.isfinite(out[torch.from_numpy(ok).to(DEV)].float()).all()
