"""C-ABI contract checks that need no GPU.

The library loads, exports every function include/moe.h declares, sizes
workspaces on the host, and rejects bad arguments with the documented status
codes before anything is enqueued.  The pointers handed over here are fake
but aligned addresses; every call is built to fail validation, so no kernel
is ever launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import fine_grained_sparse_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL, SHAPE, ALIGN, WS, UNSUP = 0, 1, 2, 3, 4, 5
FAKE = 1 << 20          # 16-byte aligned, never dereferenced
FAKE_ODD = FAKE + 8     # 8-byte aligned only


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["moe_bias_quantile", "moe_bias_update", "moe_forward",
                                  "moe_forward_noalloc", "moe_forward_slice", "moe_pack_weights",
                                  "moe_router", "moe_slice_workspace_size", "moe_status_str",
                                  "moe_workspace_size"])


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(_declared()) <= exported
    # nothing else of the library's own leaks as a C symbol
    assert {s for s in exported if s.startswith("moe_")} == set(_declared())


def test_status_strings():
    L = moe.lib()
    for code in range(8):
        assert L.moe_status_str(code)
    assert L.moe_status_str(99) == b"unknown status"


def _k2(**kw):
    base = dict(T=256, d=7168, E=384, K=8, F=2048, n_shared=1, F_shared=2048,
                d_latent=0, scale=2.827, act_dtype=moe.MOE_BF16)
    base.update(kw)
    return moe.desc(**base)


def test_workspace_size_valid_and_invalid():
    assert moe.workspace_size(_k2(), True) > moe.workspace_size(_k2(), False) > 0
    assert moe.workspace_size(_k2(T=16384), True) > moe.workspace_size(_k2(T=256), True)
    assert moe.workspace_size(_k2(T=0), True) > 0
    for bad in (dict(K=0), dict(K=17), dict(E=1025), dict(K=9, E=8), dict(d=100),
                dict(F=100), dict(F_shared=65), dict(d_latent=100), dict(n_shared=-1),
                dict(T=-1), dict(n_shared=9)):
        assert moe.workspace_size(_k2(**bad), True) == 0, bad
    # router-only sizing ignores the expert fields
    assert moe.workspace_size(_k2(F=100), False) > 0
    assert moe.workspace_size(_k2(act_dtype=7), False) == 0


def _router(D, x=FAKE, W_r=FAKE, b=FAKE, idx=FAKE, w=FAKE, counts=None, ws=FAKE, nbytes=None):
    if nbytes is None:
        nbytes = moe.workspace_size(D, False)
    vp = ctypes.c_void_p
    return moe.lib().moe_router(ctypes.byref(D), vp(x), vp(W_r), vp(b), vp(idx), vp(w),
                                vp(counts), vp(ws), nbytes, None)


def test_router_rejects_bad_arguments():
    D = _k2()
    assert _router(D, x=None) == NULL
    assert _router(D, idx=None) == NULL
    assert _router(D, ws=None) == NULL
    assert _router(D, x=FAKE_ODD) == ALIGN
    assert _router(D, counts=FAKE_ODD) == ALIGN
    assert _router(D, nbytes=moe.workspace_size(D, False) - 1) == WS
    assert _router(_k2(K=17)) == SHAPE
    assert _router(_k2(E=2000)) == SHAPE
    assert _router(_k2(d=7000)) == SHAPE
    assert _router(_k2(act_dtype=3)) == UNSUP
    # group-limited choice: groups must split E, hold >= 2 experts, <= 64 groups
    assert _router(_k2(n_group=5, topk_group=2)) == SHAPE      # 384 % 5 != 0
    assert _router(_k2(n_group=128, topk_group=2)) == SHAPE    # more than 64 groups
    assert _router(_k2(n_group=8, topk_group=0)) == SHAPE
    assert _router(_k2(n_group=8, topk_group=9)) == SHAPE
    assert _router(_k2(n_group=-1)) == SHAPE
    assert _router(_k2(E=8, K=2, n_group=8, topk_group=2)) == SHAPE  # one expert per group
    assert moe.workspace_size(_k2(n_group=8, topk_group=4), True) == moe.workspace_size(_k2(), True)
    assert moe.lib().moe_router(None, None, None, None, None, None, None, None, 0, None) == NULL


def _forward(D, W=None, nbytes=None, **ptr):
    p = dict(x=FAKE, W_r=FAKE, b=FAKE, out=FAKE, ws=FAKE)
    p.update(ptr)
    if W is None:
        W = moe.ExpertWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    if nbytes is None:
        nbytes = moe.workspace_size(D, True)
    vp = ctypes.c_void_p
    return moe.lib().moe_forward(ctypes.byref(D), vp(p["x"]), vp(p["W_r"]), vp(p["b"]),
                                 ctypes.byref(W), vp(p["out"]), vp(p.get("idx")),
                                 vp(p.get("w")), vp(p.get("counts")), vp(p.get("offsets")),
                                 vp(p.get("sorted")), vp(p["ws"]), nbytes, None, None)


def test_forward_rejects_bad_arguments():
    D = _k2()
    assert _forward(D, out=None) == NULL
    assert _forward(D, W=moe.ExpertWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None)) == NULL
    # shared weights required when n_shared > 0, latent maps when d_latent > 0
    assert _forward(D, W=moe.ExpertWeights(FAKE, FAKE, FAKE, None, None, None, None, None)) == NULL
    assert _forward(_k2(d_latent=3584)) == NULL
    assert _forward(D, W=moe.ExpertWeights(FAKE, FAKE, FAKE_ODD, FAKE, FAKE, FAKE, None, None)) == ALIGN
    assert _forward(D, sorted=FAKE_ODD) == ALIGN
    assert _forward(D, nbytes=moe.workspace_size(D, True) - 256) == WS
    assert _forward(_k2(w_dtype=moe.MOE_F32)) == UNSUP
    assert _forward(_k2(F=2000)) == SHAPE
    assert _forward(_k2(n_shared=1, F_shared=0)) == SHAPE
    # the packed layout is bf16-only; unknown layouts are refused
    assert _forward(_k2(act_dtype=moe.MOE_F32, w_layout=moe.MOE_LAYOUT_FRAG16)) == UNSUP
    assert _forward(_k2(w_layout=7)) == UNSUP
    assert _forward(_k2(w_layout=moe.MOE_LAYOUT_FRAG16), out=None) == NULL


def test_forward_rejects_bad_fp8_arguments():
    f8 = dict(w_dtype=moe.MOE_FP8_E4M3, w_layout=moe.MOE_LAYOUT_FRAG16)
    S = (FAKE, FAKE, FAKE)
    W = lambda *scales: moe.ExpertWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, *scales)  # noqa: E731
    assert moe.workspace_size(_k2(**f8), True) > 0
    # FP8 weights need bf16 activations and the packed layout
    assert _forward(_k2(w_dtype=moe.MOE_FP8_E4M3), W=W(*S)) == UNSUP
    assert _forward(_k2(act_dtype=moe.MOE_F32, **f8), W=W(*S)) == UNSUP
    # whole 128 x 128 scale blocks, K <= 8192 per projection
    assert _forward(_k2(F=2112, **f8), W=W(*S)) == SHAPE
    assert _forward(_k2(d_latent=3520, **f8), W=W(*S)) == SHAPE
    assert _forward(_k2(F=8320, **f8), W=W(*S)) == SHAPE
    assert _forward(_k2(d=8320, **f8), W=W(*S)) == SHAPE
    # the block scales are required
    assert _forward(_k2(**f8), W=W()) == NULL
    assert _forward(_k2(**f8), W=W(FAKE, FAKE, None)) == NULL


def _pack(D, src, dst):
    return moe.lib().moe_pack_weights(None if D is None else ctypes.byref(D),
                                      None if src is None else ctypes.byref(src),
                                      None if dst is None else ctypes.byref(dst), None)


def test_pack_weights_rejects_bad_arguments():
    D = _k2()
    W = lambda *p: moe.ExpertWeights(*p)  # noqa: E731
    far = FAKE + (1 << 40)                 # a second fake region, far from the first
    src = W(FAKE, None, None, None, None, None, None, None)
    assert _pack(None, src, src) == NULL
    assert _pack(D, None, src) == NULL
    # a source matrix needs a destination
    assert _pack(D, src, W(None, far, None, None, None, None, None, None)) == NULL
    assert _pack(D, src, W(far + 8, None, None, None, None, None, None, None)) == ALIGN
    # in place / overlapping buffers
    assert _pack(D, src, W(FAKE + 4096, None, None, None, None, None, None, None)) == SHAPE
    assert _pack(_k2(act_dtype=moe.MOE_F32), src, W(far, None, None, None, None, None, None, None)) == UNSUP
    assert _pack(_k2(F=100), src, W(far, None, None, None, None, None, None, None)) == SHAPE
    # FP8 routed experts pack in whole 128 x 128 blocks (act bf16)
    assert _pack(_k2(F=2112, w_dtype=moe.MOE_FP8_E4M3), src, W(far, None, None, None, None, None, None, None)) == SHAPE
    assert _pack(_k2(w_dtype=moe.MOE_FP8_E4M3, act_dtype=moe.MOE_F32), src,
                 W(far, None, None, None, None, None, None, None)) == UNSUP


def _slice(D, W=None, x=FAKE, idx=FAKE, w=FAKE, e0=0, E_total=384, out=FAKE, counts=None,
           offsets=None, sorted=None, ws=FAKE, nbytes=None):
    if W is None:
        W = moe.ExpertWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    if nbytes is None:
        nbytes = max(moe.slice_workspace_size(D, e0, E_total), 1)
    vp = ctypes.c_void_p
    return moe.lib().moe_forward_slice(ctypes.byref(D), ctypes.byref(W), vp(x), vp(idx), vp(w), e0,
                                       E_total, vp(out), vp(counts), vp(offsets), vp(sorted), vp(ws),
                                       nbytes, None)


def test_slice_workspace_size_valid_and_invalid():
    # 48 of 384 experts (one GPU of eight): no router buffers, fewer experts
    sl = moe.slice_workspace_size(_k2(E=48), 0, 384)
    assert 0 < sl < moe.workspace_size(_k2(), True)
    assert moe.slice_workspace_size(_k2(E=48), 336, 384) == sl
    # K may exceed the slice's experts (not the layer's)
    assert moe.slice_workspace_size(_k2(E=4, K=8), 380, 384) > 0
    assert moe.slice_workspace_size(_k2(E=4, K=9), 0, 8) == 0
    for e0, E, Et in ((-1, 48, 384), (337, 48, 384), (0, 48, 1025), (0, 48, 0), (0, 0, 384)):
        assert moe.slice_workspace_size(_k2(E=E), e0, Et) == 0, (e0, E, Et)
    assert moe.slice_workspace_size(_k2(E=48, F=100), 0, 384) == 0


def test_forward_slice_rejects_bad_arguments():
    D = _k2(E=48)
    for kw in (dict(x=None), dict(idx=None), dict(w=None), dict(out=None), dict(ws=None)):
        assert _slice(D, **kw) == NULL, kw
    assert _slice(D, W=moe.ExpertWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None)) == NULL
    assert _slice(D, W=moe.ExpertWeights(FAKE, FAKE, FAKE, None, None, None, None, None)) == NULL
    assert _slice(D, idx=FAKE_ODD) == ALIGN
    assert _slice(D, sorted=FAKE_ODD) == ALIGN
    assert _slice(D, W=moe.ExpertWeights(FAKE, FAKE, FAKE_ODD, FAKE, FAKE, FAKE, None, None)) == ALIGN
    assert _slice(D, nbytes=moe.slice_workspace_size(D, 0, 384) - 256) == WS
    assert _slice(D, e0=337) == SHAPE
    assert _slice(D, e0=-1) == SHAPE
    assert _slice(D, E_total=2000) == SHAPE
    assert _slice(_k2(E=48, F=2000)) == SHAPE
    assert _slice(_k2(E=48, w_dtype=moe.MOE_F32)) == UNSUP


def test_zero_tokens_accepts_null_data_pointers():
    # nothing to read or write: no kernel is launched without count outputs
    D = _k2(T=0)
    assert _router(D, x=None, W_r=None, b=None, idx=None, w=None, ws=None) == OK
    assert _forward(D, x=None, W_r=None, b=None, out=None, ws=None) == OK
    assert _forward(D, x=None, out=None, counts=FAKE_ODD) == ALIGN
    Ds = _k2(T=0, E=48)
    assert _slice(Ds, x=None, idx=None, w=None, out=None, ws=None) == OK
    assert _slice(Ds, x=None, out=None, counts=FAKE_ODD) == ALIGN


def test_bias_update_rejects_bad_arguments():
    vp = ctypes.c_void_p
    L = moe.lib()
    assert L.moe_bias_update(None, vp(FAKE), vp(FAKE), 1e-3, None) == NULL
    assert L.moe_bias_update(ctypes.byref(_k2()), None, vp(FAKE), 1e-3, None) == NULL
    assert L.moe_bias_update(ctypes.byref(_k2()), vp(FAKE), None, 1e-3, None) == NULL
    assert L.moe_bias_update(ctypes.byref(_k2()), vp(FAKE_ODD), vp(FAKE), 1e-3, None) == ALIGN
    assert L.moe_bias_update(ctypes.byref(_k2(E=2000)), vp(FAKE), vp(FAKE), 1e-3, None) == SHAPE


def test_bias_quantile_rejects_bad_arguments():
    vp = ctypes.c_void_p
    L = moe.lib()
    D = _k2(T=4096)
    n = moe.workspace_size(D, False)

    def q(D, x=FAKE, W=FAKE, b=FAKE, ws=FAKE, nbytes=n):
        return L.moe_bias_quantile(ctypes.byref(D), vp(x), vp(W), vp(b), vp(ws), nbytes, None)
    assert q(D, x=None) == NULL
    assert q(D, b=None) == NULL
    assert q(D, ws=None) == NULL
    assert q(D, b=FAKE_ODD) == ALIGN
    assert q(D, nbytes=n - 1) == WS
    assert q(_k2(T=0)) == SHAPE
    assert q(_k2(T=40000)) == SHAPE          # more tokens than the selection holds
    assert q(_k2(K=17)) == SHAPE

