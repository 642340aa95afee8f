"""moe_forward_noalloc (the layer with the library's fixed scratch array)
against moe_forward, both through the C ABI: the same outputs and routing
bit for bit on two calls in a row, the second with fewer tokens; a layer
too large for the array is refused before anything is enqueued; repeated
calls take no device memory."""
import pytest
import torch

import fine_grained_sparse_amd as moe
from moe_inputs import Workload, get_workload, make_layer_inputs
from parity import expert_weights, log, random_layer, weights_to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _same(wl, dev, w, T):
    x = dev["x"][:T].contiguous()
    ref, rr = moe.forward(x, dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=wl.n_shared,
                          return_routing=True)
    out = torch.full_like(ref, 7.0)
    got, rg = moe.forward_noalloc(x, dev["W_r"], dev["b"], w, wl.K, wl.scale,
                                  n_shared=wl.n_shared, out=out, return_routing=True)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref), T
    for k in ("idx", "w", "counts", "offsets"):
        assert torch.equal(rg[k], rr[k]), (T, k)
    assert torch.equal(rg["sorted_token"][:T * wl.K], rr["sorted_token"][:T * wl.K]), T


@pytest.mark.parametrize("name,packed", [("mid_bf16_t300", True), ("mid_bf16_t300", False),
                                         ("mid_fp8_t300", True), ("mid_latent_t200", True)])
def test_noalloc_matches_forward_small(name, packed):
    wl = get_workload(name)
    log(f"[gpu] noalloc {name} {'packed' if packed else 'rows'}: T={wl.T}, then T=77, then T=0")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=42), DEV)
    w = expert_weights(dev)
    if packed:
        w = moe.pack_weights(w, n_shared=wl.n_shared)
    _same(wl, dev, w, wl.T)
    _same(wl, dev, w, 77)          # the second call, smaller: the array keeps the first's bytes
    _same(wl, dev, w, 0)


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 6, 10, 29])
def test_noalloc_matches_forward_random_layers(seed):
    # the seeded random layers of the parity tests (all four modes, 16- and
    # 128-row tiles, latent layers), then a third of their tokens
    kw, packed, hot = random_layer(seed)
    wl = Workload(**kw)
    log(f"[gpu] noalloc {wl.name} T={wl.T} d={wl.d} E={wl.E} K={wl.K} F={wl.F} "
        f"d_latent={wl.d_latent}, then T={wl.T // 3}")
    inp = make_layer_inputs(wl, "cpu", seed=100 + seed)
    if hot is not None:
        inp["b"][hot] = 10.0
    dev = weights_to_device(inp, DEV)
    w = expert_weights(dev)
    if packed:
        w = moe.pack_weights(w, n_shared=wl.n_shared)
    _same(wl, dev, w, wl.T)
    _same(wl, dev, w, wl.T // 3)


def test_noalloc_matches_forward_k2_decode():
    wl = get_workload("k2_decode_t256")
    log("[gpu] noalloc k2_decode_t256 packed: T=256, then T=100")
    dev = make_layer_inputs(wl, DEV, seed=42)
    w = moe.pack_weights(expert_weights(dev), n_shared=wl.n_shared)
    assert moe.workspace_size(moe.desc(T=256, d=wl.d, E=wl.E, K=wl.K, F=wl.F, n_shared=1,
                                       F_shared=wl.F_shared), True) <= moe.NOALLOC_SCRATCH_BYTES
    _same(wl, dev, w, 256)
    _same(wl, dev, w, 100)
    del dev, w
    torch.cuda.empty_cache()


def test_noalloc_refuses_a_layer_beyond_its_scratch():
    wl = get_workload("mid_bf16_t300")
    T = 20000
    log(f"[gpu] noalloc refuses T={T} of mid_bf16_t300")
    inp = make_layer_inputs(wl, "cpu", seed=1)
    dev = weights_to_device(inp, DEV)
    x = torch.randn(T, wl.d, device=DEV).to(torch.bfloat16)
    D = moe.desc(T=T, d=wl.d, E=wl.E, K=wl.K, F=wl.F, n_shared=1, F_shared=wl.F_shared)
    assert moe.workspace_size(D, True) > moe.NOALLOC_SCRATCH_BYTES
    out = torch.full((T, wl.d), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.forward_noalloc(x, dev["W_r"], dev["b"], expert_weights(dev), wl.K, wl.scale,
                            n_shared=1, out=out)
    assert e.value.status == moe.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())        # nothing was enqueued


def test_noalloc_calls_take_no_device_memory():
    wl = get_workload("mid_bf16_t300")
    log("[gpu] noalloc: device memory before and after 20 calls")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=42), DEV)
    w = moe.pack_weights(expert_weights(dev), n_shared=wl.n_shared)
    out = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device=DEV)
    moe.forward_noalloc(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=1, out=out)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(20):
        moe.forward_noalloc(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=1, out=out)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_noalloc_captured_in_a_graph():
    # The use it exists for: the call captured into a HIP graph (no
    # allocation may happen under capture) and replayed, with eager work in
    # between, gives moe_forward's bits on every replay.
    wl = get_workload("mid_bf16_t300")
    log("[gpu] noalloc under graph capture, mid_bf16_t300")
    dev = weights_to_device(make_layer_inputs(wl, "cpu", seed=42), DEV)
    w = moe.pack_weights(expert_weights(dev), n_shared=wl.n_shared)
    ref = moe.forward(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=1)
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # first call on the device, outside the capture
        moe.forward_noalloc(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=1, out=out,
                            stream=side)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        moe.forward_noalloc(dev["x"], dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=1, out=out,
                            stream=side)
    for rep in range(3):
        out.fill_(0.0)
        moe.forward(dev["x"][:50].contiguous(), dev["W_r"], dev["b"], w, wl.K, wl.scale, n_shared=1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
