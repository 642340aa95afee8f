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
Zipf skew: a seeded permutation gives each expert a rank r in 1..E and an
offset o = 0.5 * r**-1.1 (fp32).  The offset is placed inside the inputs:
the last feature of every token is set to 1.0 and the last column of W_r to
o, so every logit of expert e gains exactly o_e without touching the layer.

Each tensor draws from its own torch.Generator seeded from (seed, stream).
The same seed gives the same values on the same device type; values made
on a GPU are copied to the host whenever the oracle needs them.
"""
import torch

STREAM = dict(x=1, W_r=2, b=3, zipf=4, W_gate=5, W_up=6, W_down=7,
              Ws_gate=8, Ws_up=9, Ws_down=10, W_lat_down=11, W_lat_up=12)

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


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
        offset = (0.5 * rank.pow(-1.1)).to(torch.float32)
        x[:, wl.d - 1] = 1.0
        W_r[:, wl.d - 1] = offset.to(dev)
    return dict(x=x.contiguous(), W_r=W_r.contiguous(), b=b.contiguous())


def _expert_stack(shape_one, n, std, dtype, g, dev):
    out = torch.empty((n,) + tuple(shape_one), dtype=dtype, device=dev)
    for e in range(n):
        out[e] = _normal(shape_one, std, dtype, g, dev)
    return out


def make_expert_weights(wl, device="cpu", seed=42):
    """Routed, shared and latent weights in the layouts listed above."""
    dev = torch.device(device)
    dt = _DT[wl.w_dtype]
    din, F = wl.d_in, wl.F
    w = {}
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
