"""Shared helpers of the GPU parity tests: compare the HIP path with the
CPU oracle on the same seeded inputs.

Tolerances (routing and weights as the router card's definition fixes them,
output bound derived from the arithmetic):
  * selected sets: identical, except tokens whose K-th and (K+1)-th biased
    scores (oracle, fp64) differ by less than TIE; such tokens are counted
    and the GPU's set must still be a valid top-K within TIE;
  * gate weights: |w_gpu - w_ref| <= 1e-5 |w_ref| (w_ref recomputed by the
    definition on the GPU's set where that set differs);
  * layer output: relative L2 error <= 2e-2 for bf16 experts with fp32
    accumulation (three bf16 roundings of ~2^-9 each are expected to give
    about 3e-3), <= 1e-4 for the fp32 path.
"""
import os
import sys

import numpy as np
import torch

import oracle

TIE = 1e-5
WTOL = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def effective_routing(ref, gpu_idx, gpu_w, b, K, scale):
    """Check the GPU routing against the oracle's and return the routing the
    reference output is computed with (the oracle's, or the GPU's set with
    the oracle's weights on it for near-tie tokens).

    ref: oracle.router(..., want_scores=True) result.  Returns
    (idx_eff, w_eff, stats dict)."""
    gi = np.asarray(gpu_idx)
    gw = np.asarray(gpu_w, np.float64)
    T = gi.shape[0]
    idx_eff = ref["idx"].copy()
    w_eff = ref["w"].copy()
    s = ref["scores"]
    v = s + np.asarray(b, np.float64)[None, :]
    scale64 = float(np.float32(scale))
    near = ref["gap"] < TIE
    differ = np.any(gi != ref["idx"], axis=1)
    assert not np.any(differ & ~near), (
        f"{int(np.sum(differ & ~near))} tokens select a different set with a "
        f"margin >= {TIE}: first {np.nonzero(differ & ~near)[0][:5]}")
    for t in np.nonzero(differ)[0]:
        sel = gi[t]
        assert np.all(np.diff(sel) > 0), f"token {t}: GPU slots not ascending {sel}"
        vk = np.sort(v[t])[::-1][K - 1]
        assert np.all(v[t, sel] >= vk - TIE), f"token {t}: GPU set is not a top-K within {TIE}"
        den = s[t, sel].sum() + 1e-20
        idx_eff[t] = sel
        w_eff[t] = s[t, sel] / den * scale64
    err = np.abs(gw - w_eff) / np.abs(w_eff)
    assert err.max() <= WTOL, f"gate weight rel err {err.max():.3g} > {WTOL}"
    return idx_eff, w_eff, dict(near_tie=int(near.sum()), differ=int(differ.sum()),
                                w_max_rel=float(err.max()))


def check_dispatch(gpu_routing, E):
    """Dispatch is integer work: on the GPU's own routing the oracle's
    histogram, scan and stable permutation must match bit for bit."""
    gi = gpu_routing["idx"].cpu().numpy()
    ref = oracle.dispatch(gi, E)
    np.testing.assert_array_equal(gpu_routing["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(gpu_routing["offsets"].cpu().numpy(), ref["offsets"])
    A = gi.size
    np.testing.assert_array_equal(gpu_routing["sorted_token"].cpu().numpy()[:A], ref["sorted_token"])
    return ref


def host(t):
    return t.detach().to("cpu").contiguous()


def weights_to_device(inp, device):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def expert_weights(inp):
    w = {k: inp.get(k) for k in ("W_gate", "W_up", "W_down", "Ws_gate", "Ws_up",
                                 "Ws_down", "W_lat_down", "W_lat_up")}
    for k in ("W_gate_scale", "W_up_scale", "W_down_scale"):   # FP8 routed experts
        if inp.get(k) is not None:
            w[k] = inp[k]
    return w


def frag16_reference(w):
    """include/moe.h MOE_LAYOUT_FRAG16 of [..., R, C] as a reshape/permute:
    block (i, j) of 16 rows x 32 columns at element (i * C/32 + j) * 512,
    element (r, c) of a block at ((c / 8) * 16 + r) * 8 + c % 8."""
    *lead, R, C = w.shape
    v = w.reshape(*lead, R // 16, 16, C // 32, 4, 8)
    n = len(lead)
    perm = list(range(n)) + [n + 0, n + 2, n + 3, n + 1, n + 4]   # (i, j, c/8, r, c%8)
    return v.permute(*perm).reshape(w.shape)


def frag16_fp8_reference(w):
    """include/moe.h MOE_LAYOUT_FRAG16 of an FP8 [..., R, C] as a reshape /
    permute: block (i, j) of 16 rows x 64 columns at byte (i * C/64 + j) *
    1024, element (r, c) of a block at byte (((c % 32) / 8) * 16 + r) * 16 +
    (c / 32) * 8 + c % 8."""
    *lead, R, C = w.shape
    v = w.reshape(*lead, R // 16, 16, C // 64, 2, 4, 8)   # (i, r, j, c/32, (c%32)/8, c%8)
    n = len(lead)
    perm = list(range(n)) + [n + 0, n + 2, n + 4, n + 1, n + 3, n + 5]
    return v.permute(*perm).reshape(w.shape)


def effective_routing_grouped(ref, gpu_idx, gpu_w, K, scale):
    """effective_routing for the group-limited choice.  A token is near a tie
    when its K-th / (K+1)-th masked values or its last kept / first dropped
    group scores (oracle, fp64) differ by less than TIE; only such tokens may
    differ, and then the GPU set must be K distinct ascending ids whose
    weights follow the definition on that set."""
    gi = np.asarray(gpu_idx)
    gw = np.asarray(gpu_w, np.float64)
    E = ref["scores"].shape[1]
    idx_eff = ref["idx"].copy()
    w_eff = ref["w"].copy()
    s = ref["scores"]
    scale64 = float(np.float32(scale))
    near = (ref["gap"] < TIE) | (ref["group_gap"] < TIE)
    differ = np.any(gi != ref["idx"], axis=1)
    assert not np.any(differ & ~near), (
        f"{int(np.sum(differ & ~near))} tokens select a different set with margins >= {TIE}: "
        f"first {np.nonzero(differ & ~near)[0][:5]}")
    for t in np.nonzero(differ)[0]:
        sel = gi[t]
        assert np.all(np.diff(sel) > 0) and sel.min() >= 0 and sel.max() < E, f"token {t}: {sel}"
        idx_eff[t] = sel
        w_eff[t] = s[t, sel] / (s[t, sel].sum() + 1e-20) * scale64
    err = np.abs(gw - w_eff) / np.abs(w_eff)
    assert err.max() <= WTOL, f"gate weight rel err {err.max():.3g} > {WTOL}"
    return idx_eff, w_eff, dict(near_tie=int(near.sum()), differ=int(differ.sum()),
                                w_max_rel=float(err.max()))


# ---------------------------------------------------------------- layer output
# Budget of one output element (bf16 experts, fp32 accumulation).  The GPU
# rounds the intermediates (H, the expert outputs Y and the shared output;
# in the latent form also x_lat and the latent weighted sum R) to bf16 and
# the output once; bf16 keeps 8 significant bits, so each rounding moves a
# value by at most u = 2^-8 of itself.  An element then differs from the
# exact fp64 value by
#   * at most u |ref| from the final rounding, plus
#   * the intermediate roundings carried through the following sums.  Each
#     one is a sum of many independent errors, so it behaves like a normal
#     variable of a few 1e-3 times the token's RMS output (this is the
#     ~3e-3 relative L2 the arithmetic predicts).  Over a few million checked
#     elements the largest such deviation is about 5.5 sigma, so ~1.5e-2 RMS
#     (K2 form).  The latent form has twice as many roundings on the path
#     (x_lat, R, the shared H) and a longer chain after them.
# So |gpu - ref| <= u |ref| + beta * rms(ref of that token), with beta =
# 2^-5 (K2 form) or 2^-4 (latent form), about twice the expected maximum.
# A wrong 16-column block, a wrong row or a dropped expert moves elements by
# O(rms) and fails it.  fp32 layers: no intermediate rounding; the fp32
# accumulation error is below 1e-6 relative, so 1e-5 |ref| + 1e-4 rms.
U_BF16 = 2.0 ** -8
OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}    # relative L2 error, per token and overall

RESULTS = []     # one dict per parity case, printed by tests/conftest.py at the end


def elem_budget(act_dtype, latent):
    if act_dtype == "f32":
        return 1e-5, 1e-4
    return U_BF16, (2.0 ** -4 if latent else 2.0 ** -5)


def check_output(case, got, ref, act_dtype, latent, routing_stats=None, extra=None):
    """Compare the GPU layer output with the oracle's on the checked tokens
    (rows of got / ref): every token's relative L2 error within the layer
    tolerance, the whole set's too, and every element within its budget.
    Records the numbers for the session summary and returns them."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    tol = OUT_TOL[act_dtype]
    diff = got - ref
    rn = np.linalg.norm(ref, axis=1)
    per_tok = np.linalg.norm(diff, axis=1) / np.maximum(rn, 1e-300)
    agg = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    rel_u, beta = elem_budget(act_dtype, latent)
    rms = rn / np.sqrt(max(ref.shape[1], 1))
    budget = rel_u * np.abs(ref) + beta * rms[:, None]
    # a token whose reference is exactly zero (an expert-parallel slice with
    # none of its experts) has no budget: only an exact zero passes
    ratio = np.divide(np.abs(diff), budget, out=np.where(diff == 0, 0.0, np.inf), where=budget > 0)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else (0, 0)
    rec = dict(case=case, tokens=int(got.shape[0]), rel_l2=agg,
               tok_max=float(per_tok.max()) if per_tok.size else 0.0,
               elem_ratio=float(ratio.max()) if ratio.size else 0.0)
    if routing_stats:
        rec.update({k: routing_stats[k] for k in ("near_tie", "differ", "w_max_rel") if k in routing_stats})
    if extra:
        rec.update(extra)
    RESULTS.append(rec)
    log(f"  {case}: tokens={rec['tokens']} rel_l2={agg:.3e} token_max={rec['tok_max']:.3e} "
        f"elem/budget max={rec['elem_ratio']:.3f}" +
        (f" near_tie={rec.get('near_tie')} differ={rec.get('differ')} "
         f"w_max_rel={rec.get('w_max_rel', 0):.2e}" if routing_stats else ""))
    bad = np.nonzero(per_tok > tol)[0]
    assert bad.size == 0, (f"{bad.size} tokens above relative L2 {tol}: rows {bad[:8].tolist()}, "
                           f"max {per_tok.max():.3e}")
    assert agg <= tol, f"relative L2 {agg:.3e} > {tol}"
    assert rec["elem_ratio"] <= 1.0, (
        f"element ({int(worst[0])}, {int(worst[1])}) off by {abs(diff[worst]):.3e}, budget "
        f"{budget[worst]:.3e} (ref {ref[worst]:.4e})")
    return rec


def record_routing(case, stats, tokens):
    """Routing-only cases (router, grouped router) in the session summary."""
    RESULTS.append(dict(case=case, tokens=int(tokens), near_tie=stats["near_tie"],
                        differ=stats["differ"], w_max_rel=stats["w_max_rel"]))


def coverage_tokens(T, K, counts, offsets, sorted_token, idx_eff, gap, bm=128, n_random=512,
                    seed=0, shared=True):
    """Tokens for a sampled full-size check, chosen so that every tile of the
    grouped GEMMs holds a checked row:
      * one row of every bm-row chunk of every expert's segment of the
        expert-sorted rows (the M tiles of the routed GEMMs), and the last
        row of every expert (its ragged tail);
      * one token of every bm-token chunk (the shared experts' M tiles);
    plus every near-tie token, the first token of the hottest and of the
    coldest used expert, the last token, and n_random random tokens.
    A token covers the K expert rows it was routed to."""
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts)
    offsets = np.asarray(offsets)
    st = np.asarray(sorted_token)[: T * K]
    chosen = set(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    chosen.update(np.nonzero(np.asarray(gap) < TIE)[0].tolist())
    chosen.add(T - 1)
    nz = np.nonzero(counts > 0)[0]
    for e in (nz[np.argmax(counts[nz])], nz[np.argmin(counts[nz])]):
        chosen.add(int(st[offsets[e]]))
    # sorted position of every (token, slot): pos[t] = rows token t occupies
    covered_pos = np.zeros(T * K, bool)

    def take(t):
        chosen.add(int(t))

    def mark_all():
        toks = np.fromiter(chosen, np.int64)
        mask = np.zeros(T, bool)
        mask[toks] = True
        covered_pos[:] = mask[st]
        return mask

    mask = mark_all()
    for e in nz:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        targets = [(c, min(c + bm, hi)) for c in range(lo, hi, bm)] + [(hi - 1, hi)]
        for a, b_ in targets:
            if not covered_pos[a:b_].any():
                t = int(st[rng.integers(a, b_)])
                take(t)
                mask[t] = True
                covered_pos[mask[st]] = True
    if shared:
        for c in range(0, T, bm):
            if not mask[c:c + bm].any():
                take(int(rng.integers(c, min(c + bm, T))))
    return np.array(sorted(chosen), np.int64)


# seeded random shapes of the GPU parity tests; MOE_RANDOM_LAYERS /
# MOE_RANDOM_ROUTERS widen a run (the defaults are the committed suite)
RANDOM_LAYER_SEEDS = range(int(os.environ.get("MOE_RANDOM_LAYERS", "96")))
_RANDOM_MODES = ("bf16", "packed", "fp8", "f32")  # activations / weights of a drawn layer


def random_layer(seed):
    """A seeded random layer shape within the C ABI's limits, small enough for
    the oracle to finish in about a second: E from 1 to 1024, K from 1 to
    min(E, 16), T log-uniform over 1..1500 (so rows per expert fall on both
    sides of the switch between 16-row and 128-row expert tiles, and latent
    layers on both sides of the dense maps' switch), up to 8 shared experts,
    sometimes one hot expert (bias raised, so it takes every token).  Modes
    cycle with the seed: bf16 rows, bf16 packed, FP8 packed (sizes in whole
    128 x 128 scale blocks), fp32 rows.  Returns (Workload kwargs, packed,
    hot expert or None)."""
    rng = np.random.default_rng(7919 + seed)
    mode = _RANDOM_MODES[seed % len(_RANDOM_MODES)]
    q = 128 if mode == "fp8" else 64
    while True:
        E = int(rng.choice([1, 2, 5, 8, 16, 33, 64, 100, 257, 384, 1024]))
        K = int(rng.integers(1, min(E, 16) + 1))
        T = max(1, int(np.exp(rng.uniform(0.0, np.log(1500.0)))))
        d_latent = 0 if rng.random() < 0.6 else q * int(rng.integers(1, 384 // q + 1))
        d = (q if d_latent == 0 else 64) * int(rng.integers(1, 640 // (q if d_latent == 0 else 64) + 1))
        din = d_latent or d
        F = q * int(rng.integers(1, 512 // q + 1))
        n_shared = int(rng.choice([0, 1, 1, 2, 3, 8]))
        F_shared = 64 * int(rng.integers(1, 5)) if n_shared else 0
        flops = 6.0 * T * (K * din * F + n_shared * F_shared * d) + (4.0 * T * d * d_latent)
        if flops <= 2.5e10 and 3 * E * F * din <= 4e7 and (mode != "f32" or flops <= 3e9):
            break
    hot = int(rng.integers(0, E)) if rng.random() < 0.25 else None
    kw = dict(name=f"random{seed}_{mode}", T=T, d=d, E=E, K=K, F=F, n_shared=n_shared,
              F_shared=F_shared, d_latent=d_latent, scale=float(rng.uniform(0.5, 3.0)),
              act_dtype="f32" if mode == "f32" else "bf16",
              w_dtype={"f32": "f32", "fp8": "fp8"}.get(mode, "bf16"), bias_range=0.02,
              zipf_skew=bool(rng.random() < 0.5), router_only=False)
    return kw, mode in ("packed", "fp8"), hot


RANDOM_ROUTER_SEEDS = range(int(os.environ.get("MOE_RANDOM_ROUTERS", "64")))


def random_router(seed):
    """A seeded random router shape within the C ABI's limits: E from 1 to
    1024, K up to min(E, 16), T log-uniform over 1..16384 (both the 16-row
    and the 128 x 192 logit tiles, one to sixteen split-K planes), d in
    64-steps up to 4096, fp32 or bf16 activations, a wider bias range in a
    third of them, and in a third group-limited choice (n_group a divisor of
    E with at least two experts per group, any topk_group; K may exceed the
    kept groups' experts, so that the masked scores are chosen too).
    T·E·d stays under 4e9 for the oracle.  Returns (Workload kwargs,
    n_group, topk_group)."""
    rng = np.random.default_rng(104729 + seed)
    while True:
        E = int(rng.choice([1, 2, 3, 8, 24, 64, 100, 256, 384, 512, 896, 1024]))
        K = int(rng.integers(1, min(E, 16) + 1))
        T = max(1, int(np.exp(rng.uniform(0.0, np.log(16384.0)))))
        d = 64 * int(rng.integers(1, 65))
        if T * E * d <= 4e9:
            break
    n_group, topk_group = 1, 1
    groups = [g for g in range(2, 65) if E % g == 0 and E // g >= 2]
    if groups and rng.random() < 1 / 3:
        if rng.random() < 1 / 3:  # two experts per group, one group kept
            n_group, topk_group = max(groups), 1
        else:
            n_group = int(rng.choice(groups))
            topk_group = int(rng.integers(1, n_group + 1))
    act = "f32" if rng.random() < 0.25 else "bf16"
    kw = dict(name=f"router{seed}", T=T, d=d, E=E, K=K, F=64, n_shared=0, F_shared=0,
              d_latent=0, scale=float(rng.uniform(0.5, 3.0)), act_dtype=act, w_dtype=act,
              bias_range=float(rng.choice([0.02, 0.02, 0.5])), zipf_skew=bool(rng.random() < 0.5),
              router_only=True)
    return kw, n_group, topk_group
