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
