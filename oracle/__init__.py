"""Python access to the CPU oracle of the MoE layer forward (liboracle.so).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py may import this package.  It shares no code
with the HIP library: arguments are marshalled here with ctypes and every
step of the layer runs in oracle.c, in double precision.

Inputs may be numpy arrays or CPU torch tensors; bf16 tensors are passed as
their raw 16-bit patterns and upcast exactly inside the oracle.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
F32, BF16, FP8 = 0, 1, 2
_lib = None


class OracleError(RuntimeError):
    pass


class _Layer(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
        ("F", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("F_shared", ctypes.c_int32), ("d_latent", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("W_r", ctypes.c_void_p), ("b", ctypes.c_void_p),
        ("W_gate", ctypes.c_void_p), ("W_up", ctypes.c_void_p),
        ("W_down", ctypes.c_void_p),
        ("Ws_gate", ctypes.c_void_p), ("Ws_up", ctypes.c_void_p),
        ("Ws_down", ctypes.c_void_p),
        ("W_lat_down", ctypes.c_void_p), ("W_lat_up", ctypes.c_void_p),
        ("sw_dtype", ctypes.c_int32),
        ("W_gate_scale", ctypes.c_void_p), ("W_up_scale", ctypes.c_void_p),
        ("W_down_scale", ctypes.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.oracle_router.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp,
                                    ctypes.c_float, vp, vp, vp, vp, i32]
        L.oracle_router_grouped.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                            ctypes.c_float, vp, vp, vp, vp, vp, i32]
        L.oracle_dispatch.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_bias_update.argtypes = [i32, vp, vp, ctypes.c_float, vp]
        L.oracle_bias_quantile.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32]
        L.oracle_fp8_dequant.argtypes = [i32, i32, vp, vp, vp]
        L.oracle_forward_given_routing.argtypes = [vp, i32, vp, vp, vp, vp, i32]
        L.oracle_forward.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32]
        for f in (L.oracle_router, L.oracle_router_grouped, L.oracle_dispatch, L.oracle_bias_update,
                  L.oracle_bias_quantile, L.oracle_fp8_dequant,
                  L.oracle_forward_given_routing, L.oracle_forward):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def host_cores() -> int:
    """CPU cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def default_threads() -> int:
    """Threads of the oracle's OpenMP loops: every core of the affinity mask,
    or fewer when OMP_NUM_THREADS is set lower (a share of a shared host)."""
    n = host_cores()
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host(a, what):
    """Return (contiguous numpy array, dtype code) for a CPU tensor or array."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            if a.device.type != "cpu":
                raise OracleError(f"{what}: the oracle takes host tensors")
            a = a.contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), BF16
            if a.dtype == torch.float8_e4m3fn:
                return a.view(torch.uint8).numpy(), FP8
            if a.dtype == torch.uint8:
                return a.numpy(), None
            if a.dtype == torch.float32:
                return a.numpy(), F32
            if a.dtype == torch.int32:
                return a.numpy(), None
            if a.dtype == torch.float64:
                return a.numpy(), None
            raise OracleError(f"{what}: unsupported dtype {a.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    return a, None


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc, fn):
    if rc != 0:
        raise OracleError(f"{fn} returned {rc}")


def router(x, W_r, b, K, scale, nthreads=None, want_scores=False):
    """Router of the layer.  Returns dict(idx [T,K] int32 ascending ids,
    w [T,K] float64, gap [T] float64, scores [T,E] float64 or None)."""
    xa, xdt = _host(x, "x")
    Wa, _ = _host(W_r, "W_r")
    ba, _ = _host(b, "b")
    if Wa.dtype != np.float32 or ba.dtype != np.float32:
        raise OracleError("W_r and b are fp32")
    T, d = xa.shape
    E = Wa.shape[0]
    idx = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float64)
    gap = np.zeros((T,), np.float64)
    scores = np.zeros((T, E), np.float64) if want_scores else None
    rc = lib().oracle_router(T, d, E, K, xdt, _ptr(xa), _ptr(Wa), _ptr(ba),
                             float(scale), _ptr(idx), _ptr(w), _ptr(gap),
                             _ptr(scores), nthreads or default_threads())
    _check(rc, "oracle_router")
    return dict(idx=idx, w=w, gap=gap, scores=scores)


def router_grouped(x, W_r, b, K, scale, n_group, topk_group, nthreads=None, want_scores=False):
    """Group-limited router.  Returns dict(idx, w, gap, group_gap, scores) as
    router() plus group_gap [T] (kept-group margin, +inf if all kept)."""
    xa, xdt = _host(x, "x")
    Wa, _ = _host(W_r, "W_r")
    ba, _ = _host(b, "b")
    if Wa.dtype != np.float32 or ba.dtype != np.float32:
        raise OracleError("W_r and b are fp32")
    T, d = xa.shape
    E = Wa.shape[0]
    idx = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float64)
    gap = np.zeros((T,), np.float64)
    ggap = np.zeros((T,), np.float64)
    scores = np.zeros((T, E), np.float64) if want_scores else None
    rc = lib().oracle_router_grouped(T, d, E, K, n_group, topk_group, xdt, _ptr(xa), _ptr(Wa),
                                     _ptr(ba), float(scale), _ptr(idx), _ptr(w), _ptr(gap),
                                     _ptr(ggap), _ptr(scores), nthreads or default_threads())
    _check(rc, "oracle_router_grouped")
    return dict(idx=idx, w=w, gap=gap, group_gap=ggap, scores=scores)


def bias_update(counts, b, gamma=1e-3):
    """Aux-loss-free sign update of the selection bias from per-expert counts;
    returns the new fp32 bias (numpy)."""
    c = np.ascontiguousarray(np.asarray(counts, np.int32))
    bb = np.ascontiguousarray(np.asarray(b.numpy() if hasattr(b, "numpy") else b, np.float32))
    out = np.zeros_like(bb)
    _check(lib().oracle_bias_update(c.size, _ptr(c), _ptr(bb), float(gamma), _ptr(out)),
           "oracle_bias_update")
    return out


def bias_quantile(x, W_r, K, nthreads=None):
    """Quantile Balancing bias (see oracle.h): returns (b [E] float64,
    theta [E] float64)."""
    xa, xdt = _host(x, "x")
    Wa, _ = _host(W_r, "W_r")
    if Wa.dtype != np.float32:
        raise OracleError("W_r is fp32")
    T, d = xa.shape
    E = Wa.shape[0]
    b = np.zeros((E,), np.float64)
    theta = np.zeros((E,), np.float64)
    _check(lib().oracle_bias_quantile(T, d, E, K, xdt, _ptr(xa), _ptr(Wa), _ptr(b), _ptr(theta),
                                      nthreads or default_threads()), "oracle_bias_quantile")
    return b, theta


def dispatch(idx, E):
    """Histogram, exclusive scan and stable expert-major permutation."""
    ia = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    T, K = ia.shape
    counts = np.zeros((E,), np.int32)
    offsets = np.zeros((E + 1,), np.int32)
    sorted_token = np.zeros((T * K,), np.int32)
    pos = np.zeros((T, K), np.int32)
    rc = lib().oracle_dispatch(T, E, K, _ptr(ia), _ptr(counts), _ptr(offsets),
                               _ptr(sorted_token), _ptr(pos))
    _check(rc, "oracle_dispatch")
    return dict(counts=counts, offsets=offsets, sorted_token=sorted_token,
                pos=pos)


def fp8_dequant(codes, scales):
    """Block-scaled FP8 matrix (float8_e4m3fn or uint8 codes [rows, cols],
    uint8 E8M0 scales [rows/128, cols/128]) -> float64 [rows, cols]."""
    ca, _ = _host(codes, "codes")
    sa, _ = _host(scales, "scales")
    ca = np.ascontiguousarray(ca.view(np.uint8))
    sa = np.ascontiguousarray(np.asarray(sa, dtype=np.uint8))
    rows, cols = ca.shape
    if sa.shape != (rows // 128, cols // 128):
        raise OracleError("fp8_dequant: scales must be [rows/128, cols/128]")
    out = np.zeros((rows, cols), np.float64)
    _check(lib().oracle_fp8_dequant(rows, cols, _ptr(ca), _ptr(sa), _ptr(out)),
           "oracle_fp8_dequant")
    return out


class Layer:
    """Host-side description of one layer for the oracle.

    Routed expert weights are given either stacked ([E, F, d_in] etc.) or
    as per-expert sequences whose entries may be None for experts that no
    token of the call selects (so that only the needed experts have to be
    on the host).  They are fp32, bf16, or float8_e4m3fn codes; in the FP8
    case W_gate_scale / W_up_scale / W_down_scale give, per expert, the
    uint8 E8M0 exponents of its 128 x 128 blocks ([rows/128, cols/128]).
    The shared experts and latent maps are fp32 or bf16, one dtype for all
    of them.
    """

    def __init__(self, *, d, E, K, F, scale, W_r, b, W_gate, W_up, W_down,
                 n_shared=0, F_shared=0, Ws_gate=None, Ws_up=None,
                 Ws_down=None, d_latent=0, W_lat_down=None, W_lat_up=None,
                 act_dtype=None, w_dtype=None, W_gate_scale=None,
                 W_up_scale=None, W_down_scale=None):
        self._keep = []
        self.d, self.E, self.K, self.F = d, E, K, F
        self.scale = float(scale)
        self.n_shared, self.F_shared, self.d_latent = n_shared, F_shared, d_latent
        self.W_r, _ = _host(W_r, "W_r")
        self.b, _ = _host(b, "b")
        self._keep += [self.W_r, self.b]
        rdt, sdt = [w_dtype], [w_dtype if w_dtype != FP8 else None]

        def one(a, what, slot, allowed):
            if a is None:
                return None
            arr, dt = _host(a, what)
            if dt not in allowed:
                raise OracleError(f"{what}: unsupported weight dtype")
            if slot[0] is None:
                slot[0] = dt
            elif slot[0] != dt:
                raise OracleError(f"{what}: mixed weight dtypes")
            self._keep.append(arr)
            return arr

        def raw(a, what):
            arr, _ = _host(a, what)
            if arr.dtype != np.uint8:
                raise OracleError(f"{what}: block scales must be uint8 E8M0")
            self._keep.append(arr)
            return arr

        def table(seq, what):
            arr = (ctypes.c_void_p * E)()
            for e in range(E):
                a = seq[e] if seq is not None else None
                if a is not None:
                    arr[e] = one(a, f"{what}[{e}]", rdt, (F32, BF16, FP8)).ctypes.data
            self._keep.append(arr)
            return arr

        def scale_table(seq, what):
            arr = (ctypes.c_void_p * E)()
            for e in range(E):
                a = seq[e] if seq is not None else None
                if a is not None:
                    arr[e] = raw(a, f"{what}[{e}]").ctypes.data
            self._keep.append(arr)
            return arr

        self._tables = [table(W_gate, "W_gate"), table(W_up, "W_up"),
                        table(W_down, "W_down")]
        self._scales = [scale_table(W_gate_scale, "W_gate_scale"),
                        scale_table(W_up_scale, "W_up_scale"),
                        scale_table(W_down_scale, "W_down_scale")]
        self._shared = [one(Ws_gate, "Ws_gate", sdt, (F32, BF16)),
                        one(Ws_up, "Ws_up", sdt, (F32, BF16)),
                        one(Ws_down, "Ws_down", sdt, (F32, BF16))]
        self._latent = [one(W_lat_down, "W_lat_down", sdt, (F32, BF16)),
                        one(W_lat_up, "W_lat_up", sdt, (F32, BF16))]
        self.w_dtype = rdt[0] if rdt[0] is not None else F32
        self.sw_dtype = sdt[0] if sdt[0] is not None else F32
        if self.w_dtype != FP8:
            if sdt[0] is not None and rdt[0] is not None and sdt[0] != rdt[0]:
                raise OracleError("mixed weight dtypes")
            self.sw_dtype = self.w_dtype = rdt[0] if rdt[0] is not None else self.sw_dtype
        elif W_gate_scale is None or W_up_scale is None or W_down_scale is None:
            raise OracleError("FP8 routed weights need their block scales")
        self.act_dtype = act_dtype

    def struct(self, act_dtype):
        s = _Layer()
        s.d, s.E, s.K, s.F = self.d, self.E, self.K, self.F
        s.n_shared, s.F_shared, s.d_latent = self.n_shared, self.F_shared, self.d_latent
        s.act_dtype, s.w_dtype, s.scale = act_dtype, self.w_dtype, self.scale
        s.W_r, s.b = _ptr(self.W_r), _ptr(self.b)
        s.W_gate = ctypes.cast(self._tables[0], ctypes.c_void_p)
        s.W_up = ctypes.cast(self._tables[1], ctypes.c_void_p)
        s.W_down = ctypes.cast(self._tables[2], ctypes.c_void_p)
        s.Ws_gate, s.Ws_up, s.Ws_down = [_ptr(a) for a in self._shared]
        s.W_lat_down, s.W_lat_up = [_ptr(a) for a in self._latent]
        s.sw_dtype = self.sw_dtype
        s.W_gate_scale = ctypes.cast(self._scales[0], ctypes.c_void_p)
        s.W_up_scale = ctypes.cast(self._scales[1], ctypes.c_void_p)
        s.W_down_scale = ctypes.cast(self._scales[2], ctypes.c_void_p)
        return s


def layer_from_inputs(wl, inp, experts=None):
    """Build a Layer from a moe_inputs dict of CPU tensors.  `experts`
    (optional) restricts the routed experts handed over to that set."""
    def pick(stack):
        if stack is None:
            return None
        if experts is None:
            return [stack[e] for e in range(wl.E)]
        return [stack[e] if e in experts else None for e in range(wl.E)]
    return Layer(d=wl.d, E=wl.E, K=wl.K, F=wl.F, scale=wl.scale,
                 W_r=inp["W_r"], b=inp["b"], W_gate=pick(inp["W_gate"]),
                 W_up=pick(inp["W_up"]), W_down=pick(inp["W_down"]),
                 W_gate_scale=pick(inp.get("W_gate_scale")),
                 W_up_scale=pick(inp.get("W_up_scale")),
                 W_down_scale=pick(inp.get("W_down_scale")),
                 n_shared=wl.n_shared, F_shared=wl.F_shared,
                 Ws_gate=inp.get("Ws_gate"), Ws_up=inp.get("Ws_up"),
                 Ws_down=inp.get("Ws_down"), d_latent=wl.d_latent,
                 W_lat_down=inp.get("W_lat_down"), W_lat_up=inp.get("W_lat_up"))


def forward_given_routing(layer, x, idx, w, nthreads=None):
    """Expert part of the layer for the given routing.  Returns out [T, d]
    float64."""
    xa, xdt = _host(x, "x")
    ia = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    wa = np.ascontiguousarray(np.asarray(w, dtype=np.float64))
    T = xa.shape[0]
    out = np.zeros((T, layer.d), np.float64)
    s = layer.struct(xdt)
    rc = lib().oracle_forward_given_routing(ctypes.byref(s), T, _ptr(xa),
                                            _ptr(ia), _ptr(wa), _ptr(out),
                                            nthreads or default_threads())
    _check(rc, "oracle_forward_given_routing")
    return out


def forward(layer, x, nthreads=None):
    """Whole layer.  Returns dict(out [T,d] float64, idx, w, gap)."""
    xa, xdt = _host(x, "x")
    T = xa.shape[0]
    out = np.zeros((T, layer.d), np.float64)
    idx = np.zeros((T, layer.K), np.int32)
    w = np.zeros((T, layer.K), np.float64)
    gap = np.zeros((T,), np.float64)
    s = layer.struct(xdt)
    rc = lib().oracle_forward(ctypes.byref(s), T, _ptr(xa), _ptr(out),
                              _ptr(idx), _ptr(w), _ptr(gap),
                              nthreads or default_threads())
    _check(rc, "oracle_forward")
    return dict(out=out, idx=idx, w=w, gap=gap)
