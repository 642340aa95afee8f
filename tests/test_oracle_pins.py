"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own loops: each checks a closed form,
a brute-force enumeration, a special case that reduces to a library
routine, an invariant of the definition, or a number printed on a page
(tests/golden/).  Sources:
  Kimi K2 router card (OpenModelAtlas "Kimi K2 · Router": four-step
  formula, in/out shapes, parameter table, MoEGate excerpt);
  llm-arch-kb "Kimi K2 MoE" sections 2-3 (sigmoid gate, biased top-K for
  selection only, unbiased renormalised weights, SwiGLU experts, shared
  expert added unweighted);
  lilting.ch K3 essay (latent compression 7168->3584, two shared experts).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as Fn

import oracle
from moe_inputs import Workload, get_workload, make_layer_inputs, make_router_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE32 = float(np.float32(2.827))  # the boundary takes the scale as fp32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _small(**kw):
    base = dict(name="pin", T=16, d=64, E=8, K=2, F=64, n_shared=1,
                F_shared=64, d_latent=0, scale=2.827, act_dtype="f32",
                w_dtype="f32", bias_range=0.02, zipf_skew=False,
                router_only=False)
    base.update(kw)
    return Workload(**base)


def _f32(a):
    return torch.tensor(np.asarray(a, dtype=np.float32))


# --------------------------------------------------------------------------
# Router: hand-derived worked example (closed forms, P3 four steps)
# --------------------------------------------------------------------------
def test_router_worked_example_closed_form():
    # x = e_0, so z_e = W_r[e, 0].  sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2,
    # sigmoid(-ln 3) = 1/4.  With b = (0, .3, 0, -.1):
    #   s = (.75, .5, .25, .75), v = s + b = (.75, .8, .25, .65)
    # top-2 of v = {1, 0}; without the bias it would be {0, 3}.
    # Weights use the UNBIASED s: w = 2.827 * (.75, .5) / 1.25.
    ln3 = math.log(3.0)
    x = _f32([[1.0, 0.0]])
    W_r = _f32([[ln3, 5.0], [0.0, -5.0], [-ln3, 7.0], [ln3, 1.0]])
    b = _f32([0.0, 0.3, 0.0, -0.1])
    r = oracle.router(x, W_r, b, 2, 2.827, want_scores=True)
    assert r["idx"].tolist() == [[0, 1]]
    np.testing.assert_allclose(r["scores"][0], [0.75, 0.5, 0.25, 0.75], rtol=1e-6)
    np.testing.assert_allclose(r["w"][0], [SCALE32 * 0.6, SCALE32 * 0.4], rtol=1e-6)
    np.testing.assert_allclose(r["gap"][0], 0.75 - (0.75 - 0.1), rtol=1e-5)


def test_swiglu_worked_example_closed_form():
    # One expert, d = 2, F = 1, x = e_0, K = 1 (w = scale), no shared expert.
    # g = ln 3, u = 2, h = silu(g) * u = (3/4 ln 3) * 2 = 1.5 ln 3,
    # y = W_down h with W_down = (1, -2)^T: y = (1.5 ln 3, -3 ln 3).
    ln3 = math.log(3.0)
    lay = oracle.Layer(d=2, E=1, K=1, F=1, scale=2.827, W_r=_f32([[0.0, 0.0]]),
                       b=_f32([0.0]), W_gate=[_f32([[ln3, 9.0]])],
                       W_up=[_f32([[2.0, -4.0]])], W_down=[_f32([[1.0], [-2.0]])])
    out = oracle.forward(lay, _f32([[1.0, 0.0]]))["out"][0]
    np.testing.assert_allclose(out, [SCALE32 * 1.5 * ln3, SCALE32 * -3.0 * ln3], rtol=1e-6)


# --------------------------------------------------------------------------
# Selection: brute force over every K-subset (tiny workload)
# --------------------------------------------------------------------------
def test_selection_matches_bruteforce_over_all_subsets():
    wl = get_workload("tiny_fp32_t128")
    inp = make_router_inputs(wl, "cpu", seed=7)
    r = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale, want_scores=True)
    v = r["scores"] + inp["b"].double().numpy()[None, :]
    subsets = np.array(list(itertools.combinations(range(wl.E), wl.K)))
    assert len(subsets) == math.comb(32, 4) == 35960
    M = np.zeros((len(subsets), wl.E))
    M[np.arange(len(subsets))[:, None], subsets] = 1.0
    sums = v @ M.T                                    # [T, C(E,K)]
    best = np.argmax(sums, axis=1)
    top2 = np.sort(sums, axis=1)[:, -2:]
    assert np.all(top2[:, 1] - top2[:, 0] > 1e-12)   # unique maximiser
    np.testing.assert_array_equal(r["idx"], subsets[best])


# --------------------------------------------------------------------------
# Weights: closed forms from the formula (P3) and the explanation (P3)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_fp32_t128", "mid_bf16_t300"])
def test_weights_sum_to_scale_and_G_is_zero_off_the_set(name):
    wl = get_workload(name)
    inp = make_router_inputs(wl, "cpu", seed=3)
    r = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale)
    idx, w = r["idx"], r["w"]
    np.testing.assert_allclose(w.sum(1), float(np.float32(wl.scale)), rtol=1e-12)
    assert np.all(np.diff(idx, axis=1) > 0)          # K distinct, ascending
    assert np.all((idx >= 0) & (idx < wl.E))
    G = np.zeros((wl.T, wl.E))
    np.put_along_axis(G, idx, w, axis=1)
    assert np.all((G > 0).sum(1) == wl.K)
    assert np.all((G == 0).sum(1) == wl.E - wl.K)


def test_k2_card_shapes_and_376_zeros():
    card = _golden("k2_router_card.json")
    wl = get_workload("k2_router_t4096")
    assert (wl.d, wl.E, wl.K, wl.scale) == (card["hidden_size"], card["n_routed_experts"],
                                            card["top_k"], card["routed_scaling_factor"])
    inp = make_router_inputs(wl, "cpu", seed=11, T=4)
    # parameter table: W_r [E, d] plus b [E]
    assert inp["W_r"].numel() == card["params_expert_scores"]
    assert inp["b"].numel() == card["params_select_bias"]
    assert inp["W_r"].numel() + inp["b"].numel() == card["params_per_instance"]
    assert card["params_per_instance"] * card["moe_blocks"] == card["params_all_moe_blocks"]
    r = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale)
    G = np.zeros((4, wl.E))
    np.put_along_axis(G, r["idx"], r["w"], axis=1)
    assert np.all((G == 0).sum(1) == card["zeros_per_token_in_G"])
    np.testing.assert_allclose(G.sum(1), float(np.float32(card["routed_scaling_factor"])),
                               rtol=1e-12)


def test_k3_workload_matches_k3_table():
    tab = _golden("k3_dimensions.json")
    wl = get_workload("k3_latent_t4096")
    assert (wl.d, wl.E, wl.K, wl.n_shared, wl.d_latent, wl.F, wl.F_shared) == (
        tab["hidden_size"], tab["n_routed_experts"], tab["top_k"],
        tab["n_shared_experts"], tab["latent_dim"], tab["intermediate_dim"],
        tab["intermediate_dim"])


def test_k2_expert_width_consistent_with_parameter_accounting():
    acc = _golden("k2_kb_accounting.json")
    wl = get_workload("k2_decode_t256")
    card = _golden("k2_router_card.json")
    per_expert = 3 * wl.d * wl.F
    routed_all = acc["n_routed_experts"] * per_expert * card["moe_blocks"]
    active_moe = (acc["top_k"] + acc["n_shared_experts"]) * per_expert * card["moe_blocks"]
    # routed experts are most, but not more, of the ~1.04T total; the active
    # MoE part is most, but not more, of the ~32B active
    assert 0.9 * acc["total_params_approx"] < routed_all < acc["total_params_approx"]
    assert 0.6 * acc["active_params_approx"] < active_moe < acc["active_params_approx"]


def test_bias_selects_but_does_not_weight():
    # W_r = 0: every s = 1/2, so the selection is the top-K of b alone and
    # every weight is scale / K whatever b is (bias used only for choice).
    wl = _small(E=12, K=3, T=5)
    rng = np.random.default_rng(0)
    b = rng.permutation(np.linspace(-0.05, 0.05, 12)).astype(np.float32)
    x = _f32(rng.standard_normal((5, wl.d)))
    r = oracle.router(x, _f32(np.zeros((12, wl.d))), _f32(b), 3, 2.827, want_scores=True)
    np.testing.assert_array_equal(r["scores"], 0.5)
    expect = np.sort(np.argsort(-b)[:3])
    assert all(row.tolist() == expect.tolist() for row in r["idx"])
    np.testing.assert_allclose(r["w"], SCALE32 / 3, rtol=1e-15)


def test_ties_go_to_the_lower_expert_index():
    # W_r = 0 and b = 0: all biased scores tie, the first K experts win.
    x = _f32(np.ones((3, 16)))
    r = oracle.router(x, _f32(np.zeros((10, 16))), _f32(np.zeros(10)), 4, 2.827)
    assert r["idx"].tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(r["gap"] == 0.0)


def test_sigmoid_one_hot_and_K_equals_E():
    # x = e_j makes z_e = W_r[e, j] exactly; with K = E every expert is
    # selected and w_e = scale * sigmoid(W_r[e,j]) / sum_e' sigmoid(W_r[e',j]).
    rng = np.random.default_rng(1)
    E, d, j = 9, 32, 5
    W_r = rng.standard_normal((E, d)).astype(np.float32)
    x = np.zeros((1, d), np.float32)
    x[0, j] = 1.0
    r = oracle.router(_f32(x), _f32(W_r), _f32(np.zeros(E)), E, 2.827, want_scores=True)
    s = scipy.special.expit(W_r[:, j].astype(np.float64))
    np.testing.assert_allclose(r["scores"][0], s, rtol=1e-14)
    assert r["idx"][0].tolist() == list(range(E))
    np.testing.assert_allclose(r["w"][0], SCALE32 * s / s.sum(), rtol=1e-13)
    assert math.isinf(r["gap"][0])


def test_K_equals_one_gives_the_scale_exactly():
    wl = _small(K=1, T=20)
    inp = make_router_inputs(wl, "cpu", seed=5)
    r = oracle.router(inp["x"], inp["W_r"], inp["b"], 1, 2.827)
    assert np.all(r["w"] == SCALE32)


# --------------------------------------------------------------------------
# Experts and combine: special cases reducing to library routines
# --------------------------------------------------------------------------
def _torch_swiglu(x, Wg, Wu, Wd):
    """SwiGLU with torch's silu and matmul in float64 (library routines)."""
    return (Fn.silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T


def test_single_expert_layer_reduces_to_library_swiglu():
    wl = _small(E=1, K=1, T=9, d=96, F=64, F_shared=128)
    inp = make_layer_inputs(wl, "cpu", seed=9)
    lay = oracle.layer_from_inputs(wl, inp)
    out = oracle.forward(lay, inp["x"])["out"]
    x = inp["x"].double()
    routed = _torch_swiglu(x, inp["W_gate"][0].double(), inp["W_up"][0].double(),
                           inp["W_down"][0].double())
    shared = _torch_swiglu(x, inp["Ws_gate"].double(), inp["Ws_up"].double(),
                           inp["Ws_down"].double())
    expect = shared + SCALE32 * routed
    np.testing.assert_allclose(out, expect.numpy(), rtol=1e-11, atol=1e-12)


def test_identical_experts_give_shared_plus_scale_times_expert():
    wl = _small(E=6, K=3, T=11)
    inp = make_layer_inputs(wl, "cpu", seed=4)
    for k in ("W_gate", "W_up", "W_down"):
        inp[k] = inp[k][:1].repeat(wl.E, 1, 1).contiguous()
    out = oracle.forward(oracle.layer_from_inputs(wl, inp), inp["x"])["out"]
    x = inp["x"].double()
    routed = _torch_swiglu(x, inp["W_gate"][0].double(), inp["W_up"][0].double(),
                           inp["W_down"][0].double())
    shared = _torch_swiglu(x, inp["Ws_gate"].double(), inp["Ws_up"].double(),
                           inp["Ws_down"].double())
    np.testing.assert_allclose(out, (shared + SCALE32 * routed).numpy(), rtol=1e-10, atol=1e-12)


def test_zero_down_projection_leaves_the_shared_expert_and_is_linear():
    wl = _small(E=7, K=2, T=13)
    inp = make_layer_inputs(wl, "cpu", seed=12)
    x = inp["x"]
    base = oracle.forward(oracle.layer_from_inputs(wl, inp), x)["out"]
    shared = _torch_swiglu(x.double(), inp["Ws_gate"].double(), inp["Ws_up"].double(),
                           inp["Ws_down"].double()).numpy()
    zero = dict(inp, W_down=torch.zeros_like(inp["W_down"]))
    np.testing.assert_allclose(oracle.forward(oracle.layer_from_inputs(wl, zero), x)["out"],
                               shared, rtol=1e-12, atol=1e-13)
    dbl = dict(inp, W_down=(inp["W_down"] * 2).contiguous())   # exact in fp32
    out2 = oracle.forward(oracle.layer_from_inputs(wl, dbl), x)["out"]
    np.testing.assert_allclose(out2 - shared, 2 * (base - shared), rtol=1e-10, atol=1e-12)


def test_no_shared_expert_and_only_shared_expert():
    wl = _small(E=5, K=2, T=6, n_shared=0, F_shared=0)
    inp = make_layer_inputs(wl, "cpu", seed=21)
    lay = oracle.layer_from_inputs(wl, inp)
    r = oracle.forward(lay, inp["x"])
    # without a shared expert the output is exactly the weighted routed sum
    x = inp["x"].double()
    expect = torch.zeros(wl.T, wl.d, dtype=torch.float64)
    for t in range(wl.T):
        for k in range(wl.K):
            e = int(r["idx"][t, k])
            expect[t] += r["w"][t, k] * _torch_swiglu(
                x[t:t + 1], inp["W_gate"][e].double(), inp["W_up"][e].double(),
                inp["W_down"][e].double())[0]
    np.testing.assert_allclose(r["out"], expect.numpy(), rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Dispatch: invariants and brute-force counts
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_fp32_t128", "mid_bf16_t300"])
def test_dispatch_invariants(name):
    wl = get_workload(name)
    inp = make_router_inputs(wl, "cpu", seed=2)
    idx = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale)["idx"]
    dsp = oracle.dispatch(idx, wl.E)
    counts, offsets, st, pos = dsp["counts"], dsp["offsets"], dsp["sorted_token"], dsp["pos"]
    assert counts.sum() == wl.T * wl.K
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=wl.E))
    assert offsets[0] == 0 and offsets[-1] == wl.T * wl.K
    np.testing.assert_array_equal(np.diff(offsets), counts)
    pairs = set()
    for e in range(wl.E):
        seg = st[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)               # strictly ascending tokens
        expect = np.nonzero((idx == e).any(1))[0]     # brute force membership
        np.testing.assert_array_equal(seg, expect)
        pairs.update((int(t), e) for t in seg)
    assert len(pairs) == wl.T * wl.K
    # pos is the inverse map of the permutation
    for t in range(wl.T):
        for k in range(wl.K):
            p = pos[t, k]
            assert st[p] == t and offsets[idx[t, k]] <= p < offsets[idx[t, k] + 1]


def test_dispatch_with_empty_experts():
    idx = np.array([[0, 3], [3, 5], [0, 5]], np.int32)
    dsp = oracle.dispatch(idx, 7)
    assert dsp["counts"].tolist() == [2, 0, 0, 2, 0, 2, 0]
    assert dsp["offsets"].tolist() == [0, 2, 2, 2, 4, 4, 6, 6]
    assert dsp["sorted_token"].tolist() == [0, 2, 0, 1, 1, 2]
    assert dsp["pos"].tolist() == [[0, 2], [3, 4], [1, 5]]


# --------------------------------------------------------------------------
# Layer invariants
# --------------------------------------------------------------------------
def test_tokens_are_independent():
    wl = get_workload("mid_fp32_t77")
    inp = make_layer_inputs(wl, "cpu", seed=8)
    lay = oracle.layer_from_inputs(wl, inp)
    whole = oracle.forward(lay, inp["x"])
    parts = [oracle.forward(lay, inp["x"][a:a + 20]) for a in range(0, wl.T, 20)]
    np.testing.assert_array_equal(whole["idx"], np.concatenate([p["idx"] for p in parts]))
    np.testing.assert_array_equal(whole["out"], np.concatenate([p["out"] for p in parts]))


def test_expert_relabelling_is_equivariant():
    wl = _small(E=10, K=3, T=15)
    inp = make_layer_inputs(wl, "cpu", seed=13)
    lay = oracle.layer_from_inputs(wl, inp)
    ref = oracle.forward(lay, inp["x"])
    perm = np.random.default_rng(5).permutation(wl.E)       # new label i -> old perm[i]
    p = torch.from_numpy(perm)
    inp2 = dict(inp, W_r=inp["W_r"][p].contiguous(), b=inp["b"][p].contiguous(),
                W_gate=inp["W_gate"][p].contiguous(), W_up=inp["W_up"][p].contiguous(),
                W_down=inp["W_down"][p].contiguous())
    got = oracle.forward(oracle.layer_from_inputs(wl, inp2), inp["x"])
    inv = np.argsort(perm)
    for t in range(wl.T):
        assert sorted(perm[got["idx"][t]].tolist()) == ref["idx"][t].tolist()
        wmap = dict(zip(perm[got["idx"][t]].tolist(), got["w"][t].tolist()))
        np.testing.assert_allclose([wmap[e] for e in ref["idx"][t]], ref["w"][t], rtol=1e-12)
    assert inv is not None
    np.testing.assert_allclose(got["out"], ref["out"], rtol=1e-11, atol=1e-12)


def test_latent_form_with_identity_maps_equals_plain_form():
    wl = _small(E=6, K=2, T=10, d=64)
    inp = make_layer_inputs(wl, "cpu", seed=14)
    ref = oracle.forward(oracle.layer_from_inputs(wl, inp), inp["x"])["out"]
    wl_lat = _small(E=6, K=2, T=10, d=64, d_latent=64)
    eye = torch.eye(64, dtype=torch.float32)
    inp_lat = dict(inp, W_lat_down=eye, W_lat_up=eye)
    got = oracle.forward(oracle.layer_from_inputs(wl_lat, inp_lat), inp["x"])["out"]
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_latent_form_matches_library_composition():
    wl = _small(E=1, K=1, T=7, d=96, d_latent=32, F=48, n_shared=2, F_shared=40)
    inp = make_layer_inputs(wl, "cpu", seed=15)
    out = oracle.forward(oracle.layer_from_inputs(wl, inp), inp["x"])["out"]
    x = inp["x"].double()
    xl = x @ inp["W_lat_down"].double().T
    routed = _torch_swiglu(xl, inp["W_gate"][0].double(), inp["W_up"][0].double(),
                           inp["W_down"][0].double()) @ inp["W_lat_up"].double().T
    Wg, Wu, Wd = (inp[k].double() for k in ("Ws_gate", "Ws_up", "Ws_down"))
    shared = (_torch_swiglu(x, Wg[:40], Wu[:40], Wd[:, :40]) +
              _torch_swiglu(x, Wg[40:], Wu[40:], Wd[:, 40:]))
    np.testing.assert_allclose(out, (shared + SCALE32 * routed).numpy(), rtol=1e-11, atol=1e-12)


def test_two_shared_experts_equal_one_of_double_width():
    wl2 = _small(E=4, K=2, T=8, n_shared=2, F_shared=32)
    inp = make_layer_inputs(wl2, "cpu", seed=16)
    two = oracle.forward(oracle.layer_from_inputs(wl2, inp), inp["x"])["out"]
    wl1 = _small(E=4, K=2, T=8, n_shared=1, F_shared=64)
    one = oracle.forward(oracle.layer_from_inputs(wl1, inp), inp["x"])["out"]
    np.testing.assert_allclose(two, one, rtol=1e-12, atol=1e-13)


def test_bf16_inputs_are_upcast_exactly():
    # the same values given as bf16 or as fp32 give bit-identical results
    wl = get_workload("mid_bf16_t300").with_tokens(12)
    inp = make_layer_inputs(wl, "cpu", seed=17)
    lay = oracle.layer_from_inputs(wl, inp)
    a = oracle.forward(lay, inp["x"])
    inp32 = {k: (v.float() if isinstance(v, torch.Tensor) and v.dtype == torch.bfloat16 else v)
             for k, v in inp.items()}
    b = oracle.forward(oracle.layer_from_inputs(wl, inp32), inp32["x"])
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["idx"], b["idx"])


def test_missing_expert_is_an_error():
    wl = _small(E=6, K=2, T=4)
    inp = make_layer_inputs(wl, "cpu", seed=18)
    r = oracle.router(inp["x"], inp["W_r"], inp["b"], wl.K, wl.scale)
    used = set(np.unique(r["idx"]).tolist())
    lay = oracle.layer_from_inputs(wl, inp, experts=used)
    oracle.forward_given_routing(lay, inp["x"], r["idx"], r["w"])   # enough
    lay2 = oracle.layer_from_inputs(wl, inp, experts=used - {min(used)})
    with pytest.raises(oracle.OracleError):
        oracle.forward_given_routing(lay2, inp["x"], r["idx"], r["w"])


# --------------------------------------------------------------------------
# Group-limited selection (router card, MoEGate excerpt, noaux_tc branch:
# group score = sum of the two largest biased scores of the group, keep
# topk_group groups, masked_fill(..., 0.0) on the others, top-K)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_fp32_t128", "mid_bf16_t300"])
def test_grouped_router_with_one_group_or_all_groups_is_the_plain_router(name):
    wl = get_workload(name)
    r = make_router_inputs(wl, "cpu", seed=11)
    plain = oracle.router(r["x"], r["W_r"], r["b"], wl.K, wl.scale)
    for n_group, topk_group in ((1, 1), (4, 4), (8, 8)):
        g = oracle.router_grouped(r["x"], r["W_r"], r["b"], wl.K, wl.scale, n_group, topk_group)
        assert np.array_equal(g["idx"], plain["idx"]), (n_group, topk_group)
        assert np.array_equal(g["w"], plain["w"]), (n_group, topk_group)
        assert np.all(np.isinf(g["group_gap"]))


def _designed_router(s_target, b):
    # x = e_0 and W_r[e, 0] = logit(s_e): sigmoid(z_e) = s_e up to the fp32
    # rounding of the logit (relative 1e-7).
    z = [math.log(p / (1.0 - p)) for p in s_target]
    x = _f32([[1.0, 0.0]])
    W_r = _f32([[zz, 3.0] for zz in z])
    return x, W_r, _f32(b)


def test_grouped_worked_example_closed_form():
    # 8 experts in 4 groups of 2, no bias: v = s.
    #   s      = (.9, .1 | .5, .5 | .8, .05 | .3, .2)
    #   groups:   1.0     1.0      .85        .5
    # topk_group = 2 keeps groups 0 and 1 (.8 in group 2 is the third best
    # expert overall but its group loses), so K = 3 picks {0, 2, 3}
    # (.9, .5, .5): w = 2.827 * (.9, .5, .5) / 1.9.  group_gap = 1.0 - .85.
    s = [0.9, 0.1, 0.5, 0.5, 0.8, 0.05, 0.3, 0.2]
    x, W_r, b = _designed_router(s, [0.0] * 8)
    g = oracle.router_grouped(x, W_r, b, 3, 2.827, 4, 2, want_scores=True)
    assert g["idx"].tolist() == [[0, 2, 3]]
    np.testing.assert_allclose(g["w"][0], SCALE32 * np.array([0.9, 0.5, 0.5]) / 1.9, rtol=1e-6)
    np.testing.assert_allclose(g["group_gap"][0], 0.15, rtol=1e-5)
    # the plain router would take expert 4 (.8) instead of 2
    p = oracle.router(x, W_r, b, 3, 2.827)
    assert p["idx"].tolist() == [[0, 2, 4]]


def test_grouped_ties_between_groups_go_to_the_lower_group():
    # W_r = 0 makes every s exactly 1/2, so v = 1/2 + b exactly; groups of 2
    # score (1 + .6 + .4, 1 + .4 + .6, 1 + .1 + .1) = (2, 2, 1.2): groups 0
    # and 1 tie, topk_group = 1 keeps group 0, and K = 2 takes {0, 1}.
    g = oracle.router_grouped(_f32([[1.0, 0.0]]), _f32([[0.0, 0.0]] * 6),
                              _f32([0.6, 0.4, 0.4, 0.6, 0.1, 0.1]), 2, 1.0, 3, 1)
    assert g["idx"].tolist() == [[0, 1]]
    assert g["group_gap"][0] == 0.0


def test_grouped_masked_experts_take_zero_not_minus_infinity():
    # Biased scores below zero inside the kept group lose to the 0.0 the
    # excerpt writes into the dropped groups (masked_fill with 0.0):
    #   s = .5 everywhere (z = 0), b = (-.6, -.7 | -.9, -.95)
    #   v = (-.1, -.2 | -.4, -.45); group scores -.3 | -.85 -> keep group 0;
    #   masked values (-.1, -.2, 0, 0): top-2 = {2, 3}, both from the
    #   dropped group, the ties at 0.0 going to the lower index.
    g = oracle.router_grouped(_f32([[1.0, 0.0]]), _f32([[0.0, 0.0]] * 4),
                              _f32([-0.6, -0.7, -0.9, -0.95]), 2, 1.0, 2, 1)
    assert g["idx"].tolist() == [[2, 3]]
    np.testing.assert_allclose(g["w"][0], [0.5, 0.5], rtol=1e-12)


def test_grouped_selection_matches_bruteforce_over_all_subsets():
    # Exhaustive search instead of rounds of arg-max: the kept groups are the
    # topk_group-subset of largest total group score, the selected experts
    # the K-subset of largest total masked value (the lexicographically
    # smallest one on equal totals, i.e. ties toward lower indices).  The
    # bias spans +-0.5 so that some biased scores are negative and the
    # 0.0 of the dropped groups matters.
    wl = _small(T=40, E=12, K=3, bias_range=0.5)
    r = make_router_inputs(wl, "cpu", seed=19)
    n_group, topk_group = 4, 2
    g = oracle.router_grouped(r["x"], r["W_r"], r["b"], wl.K, wl.scale, n_group, topk_group,
                              want_scores=True)
    s = g["scores"]
    v = s + r["b"].double().numpy()[None, :]
    per = wl.E // n_group
    for t in range(wl.T):
        gsc = [np.sort(v[t, q * per:(q + 1) * per])[-2:].sum() for q in range(n_group)]
        keep = max(itertools.combinations(range(n_group), topk_group),
                   key=lambda c: (sum(gsc[q] for q in c), [-q for q in c]))
        vm = np.array([v[t, e] if e // per in keep else 0.0 for e in range(wl.E)])
        best = max(itertools.combinations(range(wl.E), wl.K),
                   key=lambda c: (sum(vm[e] for e in c), [-e for e in c]))
        assert g["idx"][t].tolist() == list(best), t
        np.testing.assert_allclose(g["w"][t], s[t, list(best)] / s[t, list(best)].sum() * SCALE32,
                                   rtol=1e-12)


# --------------------------------------------------------------------------
# Aux-loss-free bias update (llm-arch-kb K2 entry: DeepSeek V3 schedule,
# sign only, gamma = 1e-3; K3 essay: a per-expert load-adjustment bias)
# --------------------------------------------------------------------------
def test_bias_update_closed_forms():
    g = np.float32(1e-3)
    # one overloaded expert: it loses gamma, the others gain gamma
    np.testing.assert_array_equal(oracle.bias_update([5, 1, 1, 1], np.zeros(4, np.float32)),
                                  np.array([-g, g, g, g], np.float32))
    # balanced load: nothing moves
    b = np.array([0.3, -0.2, 0.0, 1.0], np.float32)
    np.testing.assert_array_equal(oracle.bias_update([2, 2, 2, 2], b), b)
    # a fractional mean (4/3): the comparison is exact, 2 > 4/3 > 1
    np.testing.assert_array_equal(oracle.bias_update([2, 1, 1], np.zeros(3, np.float32)),
                                  np.array([-g, g, g], np.float32))
    # the new bias is the fp32 rounding of the exact sum (numpy's fp32 add is
    # correctly rounded too)
    b = np.array([1.0, 3.1e-4, -7.77], np.float32)
    np.testing.assert_array_equal(oracle.bias_update([0, 9, 0], b),
                                  np.array([b[0] + g, b[1] - g, b[2] + g], np.float32))


def test_bias_updates_balance_a_skewed_router():
    # What the update is for: repeated sign steps on a skewed router pull the
    # per-expert loads toward the mean (a flipped sign would widen the skew).
    wl = get_workload("tiny_fp32_t128")
    r = make_router_inputs(wl, "cpu", seed=3)
    W = r["W_r"].clone()
    W[:, 0] += torch.linspace(-0.6, 0.6, wl.E)   # skew: higher-numbered experts win
    x = r["x"].clone()
    x[:, 0] = 1.0
    b = np.zeros(wl.E, np.float32)

    def load_spread(bias):
        idx = oracle.router(x, W, torch.from_numpy(bias), wl.K, wl.scale)["idx"]
        c = np.bincount(idx.ravel(), minlength=wl.E)
        return c.max() / c.mean(), c

    start, _ = load_spread(b)
    for _ in range(60):
        _, c = load_spread(b)
        b = oracle.bias_update(c, b, gamma=0.02)
    end, _ = load_spread(b)
    assert start > 2.0 and end < 0.6 * start, (start, end)
    # the bias went down for the experts the skew favoured
    assert b[-4:].mean() < 0 < b[:4].mean()



# --------------------------------------------------------------------------
# Quantile Balancing (K3 essay, load-balancing paragraph), this reading:
# theta_e = the n-th largest router score of expert e over the batch with
# n = max(1, floor(T K / E)); b_e = mean(theta) - theta_e
# --------------------------------------------------------------------------
def _logit(p):
    return math.log(p / (1.0 - p))


def test_quantile_bias_closed_form():
    # E = 2, T = 4, K = 1: n = 2.  x_t = (logit s0_t, logit s1_t), W_r = I.
    #   s[:, 0] = (.9, .8, .3, .1) -> theta_0 = .8
    #   s[:, 1] = (.6, .5, .4, .2) -> theta_1 = .5;  mean .65 -> b = (-.15, .15)
    s0, s1 = [0.9, 0.8, 0.3, 0.1], [0.6, 0.5, 0.4, 0.2]
    x = _f32([[_logit(a), _logit(c)] for a, c in zip(s0, s1)])
    b, th = oracle.bias_quantile(x, _f32([[1.0, 0.0], [0.0, 1.0]]), 1)
    np.testing.assert_allclose(th, [0.8, 0.5], rtol=1e-6)
    np.testing.assert_allclose(b, [-0.15, 0.15], atol=1e-6)


def test_quantile_thresholds_are_the_order_statistics():
    # the defining property: at least n tokens score >= theta_e and fewer
    # than n score above it; and the bias sums to zero
    wl = get_workload("tiny_fp32_t128")
    r = make_router_inputs(wl, "cpu", seed=8)
    b, th = oracle.bias_quantile(r["x"], r["W_r"], wl.K)
    s = oracle.router(r["x"], r["W_r"], r["b"], wl.K, wl.scale, want_scores=True)["scores"]
    n = max(1, wl.T * wl.K // wl.E)
    assert np.all((s >= th[None, :]).sum(0) >= n)
    assert np.all((s > th[None, :]).sum(0) < n)
    assert abs(b.sum()) < 1e-12
    # a batch of every token twice keeps each threshold when T K / E is whole
    assert (wl.T * wl.K) % wl.E == 0
    x2 = torch.cat([r["x"], r["x"]])
    _, th2 = oracle.bias_quantile(x2, r["W_r"], wl.K)
    np.testing.assert_array_equal(th2, th)


def test_quantile_bias_balances_a_skewed_router():
    wl = get_workload("tiny_fp32_t128")
    r = make_router_inputs(wl, "cpu", seed=3)
    W = r["W_r"].clone()
    W[:, 0] += torch.linspace(-0.6, 0.6, wl.E)
    x = r["x"].clone()
    x[:, 0] = 1.0

    def spread(bias):
        idx = oracle.router(x, W, torch.from_numpy(np.asarray(bias, np.float32)), wl.K, wl.scale)["idx"]
        c = np.bincount(idx.ravel(), minlength=wl.E)
        return c.max() / c.mean()

    b, _ = oracle.bias_quantile(x, W, wl.K)
    before, after = spread(np.zeros(wl.E)), spread(b)
    assert before > 2.0 and after < 0.6 * before, (before, after)


# --------------------------------------------------------------------------
# FP8 routed experts.  The router card says only that the released weights
# are FP8 with block scales; the element format (OCP E4M3FN), the 128 x 128
# blocks and the E8M0 (power-of-two) scales are the oracle's reading.
# --------------------------------------------------------------------------
def test_fp8_codes_decode_as_torch_float8_e4m3fn():
    codes = torch.zeros((128, 128), dtype=torch.uint8)
    codes.view(-1)[:256] = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = oracle.fp8_dequant(codes, torch.full((1, 1), 127, dtype=torch.uint8)).reshape(-1)[:256]
    ref = codes.view(-1)[:256].view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    # closed forms of the format: largest 448, smallest subnormal 2^-9,
    # smallest normal 2^-6, 1.0 and -1.0, both zeros
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x00] == 0.0 and got[0x80] == 0.0


def test_fp8_block_scales_follow_the_128_blocks():
    # every code 1.0 (0x38): element (r, c) is 2^(s[r/128][c/128] - 127); a
    # 2 x 3 block grid catches a transposed or shifted scale index
    codes = torch.full((256, 384), 0x38, dtype=torch.uint8)
    s = torch.tensor([[120, 121, 122], [130, 131, 132]], dtype=torch.uint8)
    got = oracle.fp8_dequant(codes, s)
    expect = np.ldexp(1.0, s.numpy().astype(np.int64) - 127).repeat(128, 0).repeat(128, 1)
    np.testing.assert_array_equal(got, expect)
    # E8M0 ends: 2^-127 and 2^127; 255 is NaN
    ends = oracle.fp8_dequant(torch.full((128, 384), 0x38, dtype=torch.uint8),
                              torch.tensor([[0, 254, 255]], dtype=torch.uint8))
    assert ends[0, 0] == 2.0 ** -127 and ends[0, 128] == 2.0 ** 127 and np.isnan(ends[0, 256])


def _fp8_dequant_torch(codes, scales):
    """torch's float8_e4m3fn decoding times each block's power of two, in
    fp32 (exact for the generated exponents)."""
    sc = torch.pow(2.0, scales.to(torch.float64) - 127.0)
    sc = sc.repeat_interleave(128, -2).repeat_interleave(128, -1)
    return (codes.to(torch.float64) * sc).float().contiguous()


@pytest.mark.parametrize("latent", [False, True], ids=["k2", "latent"])
def test_fp8_layer_equals_the_layer_on_dequantised_weights(latent):
    wl = _small(E=5, K=2, T=9, d=256, F=128, n_shared=2, F_shared=64, act_dtype="bf16",
                w_dtype="fp8", d_latent=128 if latent else 0)
    inp = make_layer_inputs(wl, "cpu", seed=31)
    assert inp["W_gate"].dtype == torch.float8_e4m3fn and inp["W_down_scale"].shape == (5, wl.d_in // 128, 1)
    got = oracle.forward(oracle.layer_from_inputs(wl, inp), inp["x"])
    deq = {k: v for k, v in inp.items() if not k.endswith("_scale")}
    for k in ("W_gate", "W_up", "W_down"):
        deq[k] = _fp8_dequant_torch(inp[k], inp[k + "_scale"])
    for k in ("Ws_gate", "Ws_up", "Ws_down", "W_lat_down", "W_lat_up"):
        if deq.get(k) is not None:
            deq[k] = deq[k].float()          # bf16 -> fp32 is exact
    wl32 = Workload(**dict(wl.__dict__, w_dtype="f32"))
    ref = oracle.forward(oracle.layer_from_inputs(wl32, deq), inp["x"])
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    np.testing.assert_array_equal(got["out"], ref["out"])


def test_fp8_layer_needs_whole_blocks_and_scales():
    wl = _small(E=3, K=1, T=2, d=256, F=128, act_dtype="bf16", w_dtype="fp8")
    inp = make_layer_inputs(wl, "cpu", seed=3)
    no_scales = {k: v for k, v in inp.items() if not k.endswith("_scale")}
    with pytest.raises(oracle.OracleError):
        oracle.layer_from_inputs(wl, no_scales)
    # F = 64 is not a whole number of 128-blocks
    cut = dict(inp, W_gate=inp["W_gate"][:, :64].contiguous(), W_up=inp["W_up"][:, :64].contiguous(),
               W_down=inp["W_down"][:, :, :64].contiguous())
    lay = oracle.layer_from_inputs(Workload(**dict(wl.__dict__, F=64)), cut)
    with pytest.raises(oracle.OracleError):
        oracle.forward(lay, inp["x"])
