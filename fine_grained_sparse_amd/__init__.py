"""MI355X (gfx950) forward pass of a Kimi-K2-style fine-grained MoE layer.

Thin Python binding of libmoe.so, the C-ABI library declared in
include/moe.h.  This module only marshals arguments: it checks tensor
shapes and dtypes, allocates outputs and the workspace with torch (device
memory and streams are the only things torch is used for) and calls
moe_router / moe_forward.  Every step of the layer runs in the library's
HIP kernels; there is no fallback, and importing this module without the
built library raises.

Layer (OpenModelAtlas "Kimi K2 · Router" four steps; llm-arch-kb "Kimi K2
MoE" sections 2-3; lilting.ch K3 essay for the latent form):
    s = sigmoid(x W_r^T);  S = top_K(s + b);  w_i = scale * s_i / (sum_S s + 1e-20)
    out = sum_shared f_s(x) + U(sum_{i in S} w_i f_i(L(x)))
with SwiGLU experts f(v) = W_down (silu(W_gate v) * (W_up v)).
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_LAYOUT_ROWS, MOE_LAYOUT_FRAG16 = 0, 1
_STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
           4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_UNSUPPORTED", 6: "MOE_ERR_HIP", 7: "MOE_ERR_SCRATCH"}
MOE_ERR_SCRATCH = 7
NOALLOC_SCRATCH_BYTES = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES
_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}
EXPORTS = ("moe_workspace_size", "moe_router", "moe_forward", "moe_forward_noalloc", "moe_pack_weights",
           "moe_bias_update", "moe_bias_quantile", "moe_status_str", "moe_slice_workspace_size",
           "moe_forward_slice")
WEIGHT_NAMES = ("W_gate", "W_up", "W_down", "Ws_gate", "Ws_up", "Ws_down", "W_lat_down", "W_lat_up")
SCALE_NAMES = ("W_gate_scale", "W_up_scale", "W_down_scale")  # FP8 routed experts only
STAGES = ("start", "router", "dispatch", "latent", "up", "down", "end")
NUM_STAGE_EVENTS = len(STAGES)


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().moe_status_str(status).decode()
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({msg})")


class LayerDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("F", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("F_shared", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("scale", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("w_layout", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32)]


class ExpertWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES + SCALE_NAMES]


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "fine_grained_sparse_amd/build.py (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.moe_workspace_size.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_int]
        L.moe_workspace_size.restype = ctypes.c_size_t
        L.moe_router.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
        L.moe_router.restype = ctypes.c_int
        L.moe_forward.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, vp,
                                  ctypes.POINTER(ExpertWeights), vp, vp, vp, vp, vp, vp,
                                  vp, ctypes.c_size_t, vp, vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, vp,
                                          ctypes.POINTER(ExpertWeights), vp, vp, vp, vp, vp, vp, vp]
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_slice_workspace_size.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_int32, ctypes.c_int32]
        L.moe_slice_workspace_size.restype = ctypes.c_size_t
        L.moe_forward_slice.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(ExpertWeights), vp, vp, vp,
                                        ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                        vp]
        L.moe_forward_slice.restype = ctypes.c_int
        L.moe_pack_weights.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(ExpertWeights),
                                       ctypes.POINTER(ExpertWeights), vp]
        L.moe_pack_weights.restype = ctypes.c_int
        L.moe_bias_update.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, ctypes.c_float, vp]
        L.moe_bias_update.restype = ctypes.c_int
        L.moe_bias_quantile.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_bias_quantile.restype = ctypes.c_int
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def desc(*, T, d, E, K, F=0, n_shared=0, F_shared=0, d_latent=0, scale=2.827,
         act_dtype=MOE_BF16, w_dtype=None, w_layout=MOE_LAYOUT_ROWS, n_group=1, topk_group=1):
    return LayerDesc(T, d, E, K, F, n_shared, F_shared, d_latent, scale, act_dtype,
                     act_dtype if w_dtype is None else w_dtype, w_layout, n_group, topk_group)


def workspace_size(layer_desc: LayerDesc, forward: bool) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(layer_desc), 1 if forward else 0))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class Workspace:
    """Growable device byte buffers (allocated by torch, owned here), one per
    (device, stream).  A buffer is allocated while its stream is current, so
    torch's caching allocator orders any reuse of its memory after the work
    already queued on that stream; calls on different streams never share
    scratch, and a buffer that grows is released only in that stream's
    order."""

    def __init__(self):
        self._buf = {}

    def get(self, device, nbytes, stream=None):
        s = torch.cuda.current_stream(device) if stream is None else stream
        key = (device, s.cuda_stream)
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            self._buf.pop(key, None)
            with torch.cuda.stream(s):
                buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._buf[key] = buf
        return buf


_default_ws = Workspace()


def _on(stream):
    """Context in which outputs are allocated: the launch stream."""
    return torch.cuda.stream(stream) if stream is not None else _Nothing()


class _Nothing:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def router(x, W_r, b, K, scale=2.827, *, counts=True, workspace=None, stream=None,
           n_group=1, topk_group=1):
    """moe_router: returns (topk_idx int32 [T,K], topk_w fp32 [T,K],
    expert_counts int32 [E] or None).  Slots are in ascending expert id.
    n_group > 1 limits the choice to the topk_group best expert groups."""
    _need(x, "x")
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("x must be [T, d] fp32 or bf16")
    T, d = x.shape
    dev = x.device
    _need(W_r, "W_r", torch.float32, device=dev)
    E = W_r.shape[0]
    _need(W_r, "W_r", torch.float32, (E, d))
    _need(b, "b", torch.float32, (E,), dev)
    D = desc(T=T, d=d, E=E, K=K, scale=scale, act_dtype=_DT[x.dtype], n_group=n_group,
             topk_group=topk_group)
    nbytes = workspace_size(D, False)
    if nbytes == 0:
        raise MoeError("moe_workspace_size", 2)
    with _on(stream):
        idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
        cnt = torch.empty((E,), dtype=torch.int32, device=dev) if counts else None
    ws = (workspace or _default_ws).get(dev, nbytes, stream)
    rc = lib().moe_router(ctypes.byref(D), _ptr(x), _ptr(W_r), _ptr(b), _ptr(idx), _ptr(w),
                          _ptr(cnt), _ptr(ws), nbytes, _stream(stream))
    if rc:
        raise MoeError("moe_router", rc)
    return idx, w, cnt


def _weights_desc(weights, T, d, E, K, scale, dt, dev, n_shared, n_group=1, topk_group=1):
    """Validate the weight tensors; return (LayerDesc, ExpertWeights).
    Routed experts are of dtype dt, or float8_e4m3fn codes with uint8 E8M0
    block scales (W_gate_scale, W_up_scale [E, F/128, d_in/128];
    W_down_scale [E, d_in/128, F/128]) when dt is bf16."""
    Wg, Wu, Wd = weights["W_gate"], weights["W_up"], weights["W_down"]
    f8 = isinstance(Wg, torch.Tensor) and Wg.dtype == torch.float8_e4m3fn and dt == torch.bfloat16
    rdt = torch.float8_e4m3fn if f8 else dt
    _need(Wg, "W_gate", rdt, device=dev)
    if Wg.dim() != 3 or Wg.shape[0] != E:
        raise ValueError("W_gate must be [E, F, d_in]")
    F, din = Wg.shape[1], Wg.shape[2]
    _need(Wu, "W_up", rdt, (E, F, din), dev)
    _need(Wd, "W_down", rdt, (E, din, F), dev)
    scales = [None] * 3
    if f8:
        if F % 128 or din % 128:
            raise ValueError("FP8 routed experts need F and d_in in whole 128-blocks")
        shapes = ((E, F // 128, din // 128), (E, F // 128, din // 128), (E, din // 128, F // 128))
        for i, (n, shp) in enumerate(zip(SCALE_NAMES, shapes)):
            _need(weights.get(n), n, torch.uint8, shp, dev)
            scales[i] = weights[n]
    Wl_d, Wl_u = weights.get("W_lat_down"), weights.get("W_lat_up")
    d_lat = 0
    if Wl_d is not None or Wl_u is not None:
        d_lat = din
        _need(Wl_d, "W_lat_down", dt, (d_lat, d), dev)
        _need(Wl_u, "W_lat_up", dt, (d, d_lat), dev)
    elif din != d:
        raise ValueError("experts act on d_in != d but no latent maps were given")
    Wsg, Wsu, Wsd = weights.get("Ws_gate"), weights.get("Ws_up"), weights.get("Ws_down")
    ns = 0 if Wsg is None else (1 if n_shared is None else n_shared)
    Fs = 0
    if ns:
        if Wsg.shape[0] % ns:
            raise ValueError("Ws_gate rows must be n_shared * F_shared")
        Fs = Wsg.shape[0] // ns
        _need(Wsg, "Ws_gate", dt, (ns * Fs, d), dev)
        _need(Wsu, "Ws_up", dt, (ns * Fs, d), dev)
        _need(Wsd, "Ws_down", dt, (d, ns * Fs), dev)
    layout = int(weights.get("layout", MOE_LAYOUT_ROWS))
    D = desc(T=T, d=d, E=E, K=K, F=F, n_shared=ns, F_shared=Fs, d_latent=d_lat,
             scale=scale, act_dtype=_DT[dt], w_dtype=MOE_FP8_E4M3 if f8 else None,
             w_layout=layout, n_group=n_group, topk_group=topk_group)
    W = ExpertWeights(*[None if t is None else t.data_ptr() for t in
                        (Wg, Wu, Wd, Wsg, Wsu, Wsd, Wl_d, Wl_u, *scales)])
    return D, W


def bias_update(counts, b, gamma=1e-3, *, stream=None):
    """moe_bias_update: b (fp32 [E], in place) += gamma * sgn(mean - counts)
    from the per-expert selection counts (int32 [E]) of one or more
    batches.  Returns b."""
    _need(counts, "counts", torch.int32)
    E = counts.numel()
    _need(b, "b", torch.float32, (E,), counts.device)
    D = desc(T=0, d=64, E=E, K=1)
    rc = lib().moe_bias_update(ctypes.byref(D), _ptr(counts), _ptr(b), float(gamma), _stream(stream))
    if rc:
        raise MoeError("moe_bias_update", rc)
    return b


def bias_quantile(x, W_r, K, *, out=None, workspace=None, stream=None):
    """moe_bias_quantile: the Quantile Balancing bias of a batch (fp32 [E]):
    b_e = mean(theta) - theta_e with theta_e the n-th largest router score of
    expert e, n = max(1, T K // E)."""
    _need(x, "x")
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("x must be [T, d] fp32 or bf16")
    T, d = x.shape
    dev = x.device
    _need(W_r, "W_r", torch.float32, device=dev)
    E = W_r.shape[0]
    _need(W_r, "W_r", torch.float32, (E, d))
    D = desc(T=T, d=d, E=E, K=K, act_dtype=_DT[x.dtype])
    nbytes = workspace_size(D, False)
    if nbytes == 0:
        raise MoeError("moe_workspace_size", 2)
    with _on(stream):
        b = torch.empty((E,), dtype=torch.float32, device=dev) if out is None else out
    _need(b, "out", torch.float32, (E,), dev)
    ws = (workspace or _default_ws).get(dev, nbytes, stream)
    rc = lib().moe_bias_quantile(ctypes.byref(D), _ptr(x), _ptr(W_r), _ptr(b), _ptr(ws), nbytes,
                                 _stream(stream))
    if rc:
        raise MoeError("moe_bias_quantile", rc)
    return b


def pack_weights(weights, *, n_shared=None, stream=None):
    """moe_pack_weights: row-major weights (bf16, or FP8 routed experts with
    bf16 shared / latent maps) -> a new dict of tensors of the same shapes
    in MOE_LAYOUT_FRAG16, with "layout" set (FP8 block scales are carried
    over as they are).  Run once, e.g. at model load; the packed tensors are
    what forward() then reads."""
    if int(weights.get("layout", MOE_LAYOUT_ROWS)) != MOE_LAYOUT_ROWS:
        raise ValueError("weights are already packed")
    Wg = weights["W_gate"]
    if Wg.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError("only bf16 and FP8 weights have a packed layout")
    E, F, din = Wg.shape
    d = weights["W_lat_down"].shape[1] if weights.get("W_lat_down") is not None else din
    D, src = _weights_desc(weights, 1, d, E, 1, 1.0, torch.bfloat16, Wg.device, n_shared)
    with _on(stream):
        out = {k: (torch.empty_like(weights[k]) if weights.get(k) is not None else None)
               for k in WEIGHT_NAMES}
    dst = ExpertWeights(*[None if out[k] is None else out[k].data_ptr() for k in WEIGHT_NAMES])
    for k in SCALE_NAMES:
        if weights.get(k) is not None:
            out[k] = weights[k]
    rc = lib().moe_pack_weights(ctypes.byref(D), ctypes.byref(src), ctypes.byref(dst), _stream(stream))
    if rc:
        raise MoeError("moe_pack_weights", rc)
    out["layout"] = MOE_LAYOUT_FRAG16
    return out


def _forward_call(x, W_r, b, weights, K, scale, n_shared, out, return_routing, stream,
                  n_group, topk_group):
    """Validate and marshal the arguments of moe_forward / moe_forward_noalloc;
    outputs are allocated on the launch stream.  Returns (desc, weights
    struct, out, routing dict or None, pointer tuple of the outputs)."""
    _need(x, "x")
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("x must be [T, d] fp32 or bf16")
    T, d = x.shape
    dev, dt = x.device, x.dtype
    E = W_r.shape[0]
    _need(W_r, "W_r", torch.float32, (E, d), dev)
    _need(b, "b", torch.float32, (E,), dev)
    D, W = _weights_desc(weights, T, d, E, K, scale, dt, dev, n_shared, n_group, topk_group)
    with _on(stream):
        if out is None:
            out = torch.empty((T, d), dtype=dt, device=dev)
        routing = None
        if return_routing:
            routing = dict(idx=torch.empty((T, K), dtype=torch.int32, device=dev),
                           w=torch.empty((T, K), dtype=torch.float32, device=dev),
                           counts=torch.empty((E,), dtype=torch.int32, device=dev),
                           offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
                           sorted_token=torch.empty((max(T * K, 1),), dtype=torch.int32,
                                                    device=dev))
    _need(out, "out", dt, (T, d), dev)
    r = routing or {}
    outs = (_ptr(out), _ptr(r.get("idx")), _ptr(r.get("w")), _ptr(r.get("counts")),
            _ptr(r.get("offsets")), _ptr(r.get("sorted_token")))
    return D, W, out, routing, outs


def forward(x, W_r, b, weights, K, scale=2.827, *, n_shared=None, out=None,
            return_routing=False, workspace=None, stream=None, stage_events=None,
            n_group=1, topk_group=1):
    """moe_forward: the whole layer.  `weights` holds W_gate [E,F,d_in],
    W_up [E,F,d_in], W_down [E,d_in,F] and optionally Ws_gate/Ws_up
    [n_shared*F_shared, d], Ws_down [d, n_shared*F_shared], W_lat_down
    [d_latent, d], W_lat_up [d, d_latent], plus "layout" (MOE_LAYOUT_ROWS
    when absent; pack_weights returns MOE_LAYOUT_FRAG16 weights).  With bf16
    x the routed experts may be float8_e4m3fn codes (packed) with uint8 E8M0
    block scales W_gate_scale, W_up_scale, W_down_scale.  Returns
    out [T, d], or (out, routing dict) with return_routing=True.
    `stage_events` (optional) is a sequence of NUM_STAGE_EVENTS
    already-created torch.cuda.Event objects recorded at the stage
    boundaries listed in include/moe.h.  n_group > 1 limits the routing to
    the topk_group best expert groups (as router())."""
    D, W, out, routing, outs = _forward_call(x, W_r, b, weights, K, scale, n_shared, out,
                                             return_routing, stream, n_group, topk_group)
    nbytes = workspace_size(D, True)
    if nbytes == 0:
        raise MoeError("moe_workspace_size", 2)
    ev = None
    if stage_events is not None:
        if len(stage_events) != NUM_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {NUM_STAGE_EVENTS} events")
        ev = (ctypes.c_void_p * NUM_STAGE_EVENTS)(*[e.cuda_event or None for e in stage_events])
    ws = (workspace or _default_ws).get(x.device, nbytes, stream)
    rc = lib().moe_forward(ctypes.byref(D), _ptr(x), _ptr(W_r), _ptr(b), ctypes.byref(W), *outs,
                           _ptr(ws), nbytes, _stream(stream), ev)
    if rc:
        raise MoeError("moe_forward", rc)
    return (out, routing) if return_routing else out


def slice_workspace_size(layer_desc: LayerDesc, e0: int, E_total: int) -> int:
    return int(lib().moe_slice_workspace_size(ctypes.byref(layer_desc), e0, E_total))


def forward_slice(x, topk_idx, topk_w, weights, e0, E_total, *, n_shared=None, out=None,
                  return_dispatch=False, workspace=None, stream=None):
    """moe_forward_slice: one GPU's share of an expert-parallel layer.
    `weights` holds the slice's routed experts only (W_gate [E, F, d_in],
    ... for experts e0 .. e0 + E - 1 of E_total), plus the shared experts
    (added to every token) and latent maps as forward() takes them;
    topk_idx / topk_w [T, K] are the routing router() returned over all
    E_total experts.  Returns out [T, d], or (out, dict of counts [E],
    offsets [E + 1] and sorted_token over the slice's local experts) with
    return_dispatch=True."""
    _need(x, "x")
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("x must be [T, d] fp32 or bf16")
    T, d = x.shape
    dev, dt = x.device, x.dtype
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise ValueError("topk_idx must be [T, K]")
    K = topk_idx.shape[1]
    _need(topk_idx, "topk_idx", torch.int32, (T, K), dev)
    _need(topk_w, "topk_w", torch.float32, (T, K), dev)
    E = weights["W_gate"].shape[0]
    D, W = _weights_desc(weights, T, d, E, K, 1.0, dt, dev, n_shared)
    with _on(stream):
        if out is None:
            out = torch.empty((T, d), dtype=dt, device=dev)
        disp = None
        if return_dispatch:
            disp = dict(counts=torch.empty((E,), dtype=torch.int32, device=dev),
                        offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
                        sorted_token=torch.empty((max(T * K, 1),), dtype=torch.int32, device=dev))
    _need(out, "out", dt, (T, d), dev)
    nbytes = slice_workspace_size(D, e0, E_total)
    if nbytes == 0:
        raise MoeError("moe_slice_workspace_size", 2)
    ws = (workspace or _default_ws).get(x.device, nbytes, stream)
    r = disp or {}
    rc = lib().moe_forward_slice(ctypes.byref(D), ctypes.byref(W), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                 e0, E_total, _ptr(out), _ptr(r.get("counts")), _ptr(r.get("offsets")),
                                 _ptr(r.get("sorted_token")), _ptr(ws), nbytes, _stream(stream))
    if rc:
        raise MoeError("moe_forward_slice", rc)
    return (out, disp) if return_dispatch else out


def forward_noalloc(x, W_r, b, weights, K, scale=2.827, *, n_shared=None, out=None,
                    return_routing=False, stream=None, n_group=1, topk_group=1):
    """moe_forward_noalloc: forward() with the library's fixed scratch array
    (NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace.  The library
    allocates nothing; pass `out` (and no return_routing) for a call that
    allocates nothing here either.  Raises MoeError with status
    MOE_ERR_SCRATCH when the layer needs more scratch than the array holds.
    Calls that overlap in time on one GPU share the array and race."""
    D, W, out, routing, outs = _forward_call(x, W_r, b, weights, K, scale, n_shared, out,
                                             return_routing, stream, n_group, topk_group)
    rc = lib().moe_forward_noalloc(ctypes.byref(D), _ptr(x), _ptr(W_r), _ptr(b), ctypes.byref(W),
                                   *outs, _stream(stream))
    if rc:
        raise MoeError("moe_forward_noalloc", rc)
    return (out, routing) if return_routing else out


__all__ = ["router", "forward", "forward_noalloc", "pack_weights", "bias_update", "bias_quantile", "workspace_size", "desc", "lib", "MoeError",
           "LayerDesc", "ExpertWeights", "Workspace", "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3",
           "MOE_LAYOUT_ROWS", "MOE_LAYOUT_FRAG16", "EXPORTS", "WEIGHT_NAMES", "SCALE_NAMES"]
