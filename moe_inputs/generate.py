"""Seeded tensor generation for the MoE workloads.

Recipe (values only; nothing here computes any part of the layer):
  x        ~ N(0, 1), rounded to the activation dtype (RNE for bf16)
  W_r      ~ N(0, 1/d), fp32, layout [E, d]
  b        ~ U(-bias_range, bias_range), fp32, [E]
  W_gate, W_up ~ N(0, 1/d_in), layout [E, F, d_in]
  W_down   ~ N(0, 1/F), layout [E, d_in, F]
  Ws_gate, Ws_up ~ N(0, 1/d), [n_shared*F_shared, d] (shared experts stacked)
  Ws_down  ~ N(0, 1/F_shared), [d, n_shared*F_shared]
  W_lat_down ~ N(0, 1/d), [d_latent, d];  W_lat_up ~ N(0, 1/d_latent), [d, d_latent]
FP8 routed experts (w_dtype "fp8"; shared experts and latent maps bf16):
  each routed matrix of target std sigma = fan_in**-0.5 is drawn as
  E8M0 block exponents s = 127 + round(log2(sigma / 16)) + j, j uniform in
  {-1, 0, 1} per 128 x 128 block, and codes = float8_e4m3fn(16 * N(0, 1))
  (torch's round-to-nearest cast is only the sampler: the layer takes the
  codes as given), so code * 2^(s - 127) has std about sigma.
Zipf skew: a seeded permutation gives each expert a rank r in 1..E and an
offset o = a * r**-1.1 (fp32), a = the workload's zipf_scale (0.5 unless
stated).  The offset is placed inside the inputs:
the last feature of every token is set to 1.0 and the last column of W_r to
o, so every logit of expert e gains exactly o_e without touching the layer.

Each tensor draws from its own torch.Generator seeded from (seed, stream).
The same seed gives the same values on the same device type; values made
on a GPU are copied to the host whenever the oracle needs them.
"""
import math

import torch

STREAM = dict(x=1, W_r=2, b=3, zipf=4, W_gate=5, W_up=6, W_down=7,
              Ws_gate=8, Ws_up=9, Ws_down=10, W_lat_down=11, W_lat_up=12,
              W_gate_scale=13, W_up_scale=14, W_down_scale=15)

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
FP8_CODE_STD = 16.0


def _dense_dtype(wl):
    """dtype of the shared experts and latent maps."""
    return torch.bfloat16 if wl.w_dtype == "fp8" else _DT[wl.w_dtype]


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream)
    return g


def _normal(shape, std, dtype, g, device):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_router_inputs(wl, device="cpu", seed=42, T=None):
    """x [T, d] (activation dtype), W_r [E, d] fp32, b [E] fp32."""
    T = wl.T if T is None else T
    dev = torch.device(device)
    x = _normal((T, wl.d), 1.0, _DT[wl.act_dtype], _gen(seed, STREAM["x"], dev), dev)
    W_r = _normal((wl.E, wl.d), wl.d ** -0.5, torch.float32,
                  _gen(seed, STREAM["W_r"], dev), dev)
    u = torch.rand((wl.E,), generator=_gen(seed, STREAM["b"], dev), device=dev,
                   dtype=torch.float32)
    b = (u * 2.0 - 1.0) * wl.bias_range
    if wl.zipf_skew:
        perm = torch.randperm(wl.E, generator=_gen(seed, STREAM["zipf"], torch.device("cpu")))
        rank = (perm + 1).to(torch.float64)
        offset = (wl.zipf_scale * rank.pow(-1.1)).to(torch.float32)
        x[:, wl.d - 1] = 1.0
        W_r[:, wl.d - 1] = offset.to(dev)
    return dict(x=x.contiguous(), W_r=W_r.contiguous(), b=b.contiguous())


def _expert_stack(shape_one, n, std, dtype, g, dev):
    out = torch.empty((n,) + tuple(shape_one), dtype=dtype, device=dev)
    for e in range(n):
        out[e] = _normal(shape_one, std, dtype, g, dev)
    return out


def _fp8_stack(shape_one, n, std, g, gs, dev):
    """n block-scaled FP8 matrices: (codes float8_e4m3fn [n, r, c],
    E8M0 exponents uint8 [n, r/128, c/128])."""
    r, c = shape_one
    base = 127 + int(round(math.log2(std / FP8_CODE_STD)))
    codes = torch.empty((n, r, c), dtype=torch.float8_e4m3fn, device=dev)
    for e in range(n):
        codes[e] = _normal((r, c), FP8_CODE_STD, torch.float32, g, dev).to(torch.float8_e4m3fn)
    jit = torch.randint(-1, 2, (n, r // 128, c // 128), generator=gs, device=dev, dtype=torch.int32)
    return codes, (jit + base).to(torch.uint8)


def make_expert_weights(wl, device="cpu", seed=42):
    """Routed, shared and latent weights in the layouts listed above."""
    dev = torch.device(device)
    dt = _dense_dtype(wl)
    din, F = wl.d_in, wl.F
    w = {}
    if wl.w_dtype == "fp8":
        for name, shp, fan in (("W_gate", (F, din), din), ("W_up", (F, din), din),
                               ("W_down", (din, F), F)):
            w[name], w[name + "_scale"] = _fp8_stack(
                shp, wl.E, fan ** -0.5, _gen(seed, STREAM[name], dev),
                _gen(seed, STREAM[name + "_scale"], dev), dev)
    else:
        w["W_gate"] = _expert_stack((F, din), wl.E, din ** -0.5, dt,
                                    _gen(seed, STREAM["W_gate"], dev), dev)
        w["W_up"] = _expert_stack((F, din), wl.E, din ** -0.5, dt,
                                  _gen(seed, STREAM["W_up"], dev), dev)
        w["W_down"] = _expert_stack((din, F), wl.E, F ** -0.5, dt,
                                    _gen(seed, STREAM["W_down"], dev), dev)
    Fs = wl.n_shared * wl.F_shared
    if Fs:
        w["Ws_gate"] = _normal((Fs, wl.d), wl.d ** -0.5, dt,
                               _gen(seed, STREAM["Ws_gate"], dev), dev)
        w["Ws_up"] = _normal((Fs, wl.d), wl.d ** -0.5, dt,
                             _gen(seed, STREAM["Ws_up"], dev), dev)
        w["Ws_down"] = _normal((wl.d, Fs), wl.F_shared ** -0.5, dt,
                               _gen(seed, STREAM["Ws_down"], dev), dev)
    else:
        w["Ws_gate"] = w["Ws_up"] = w["Ws_down"] = None
    if wl.d_latent:
        w["W_lat_down"] = _normal((wl.d_latent, wl.d), wl.d ** -0.5, dt,
                                  _gen(seed, STREAM["W_lat_down"], dev), dev)
        w["W_lat_up"] = _normal((wl.d, wl.d_latent), wl.d_latent ** -0.5, dt,
                                _gen(seed, STREAM["W_lat_up"], dev), dev)
    else:
        w["W_lat_down"] = w["W_lat_up"] = None
    return w


def make_layer_inputs(wl, device="cpu", seed=42):
    d = make_router_inputs(wl, device, seed)
    if not wl.router_only:
        d.update(make_expert_weights(wl, device, seed))
    return d
