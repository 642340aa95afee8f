"""moe_pack_weights writes exactly the fragment-block layout include/moe.h
defines (a pure permutation, checked bit for bit).  The reference below is
the header's formula written as a reshape/permute: block (i, j) of 16 rows x
32 columns at element (i * cols/32 + j) * 512, element (r, c) of a block at
((c / 8) * 16 + r) * 8 + c % 8."""
import pytest
import torch

import fine_grained_sparse_amd as moe
from parity import frag16_fp8_reference, frag16_reference, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rand(shape, g):
    return (torch.randn(shape, generator=g) * 0.5).to(torch.bfloat16)


@pytest.mark.parametrize("latent", [False, True])
def test_pack_is_the_documented_permutation(latent):
    log(f"[gpu] pack layout latent={latent}")
    g = torch.Generator().manual_seed(3)
    E, F, d, dl, ns, Fs = 3, 64, 192, 128, 2, 64
    din = dl if latent else d
    w = dict(W_gate=_rand((E, F, din), g), W_up=_rand((E, F, din), g), W_down=_rand((E, din, F), g),
             Ws_gate=_rand((ns * Fs, d), g), Ws_up=_rand((ns * Fs, d), g), Ws_down=_rand((d, ns * Fs), g),
             W_lat_down=_rand((dl, d), g) if latent else None, W_lat_up=_rand((d, dl), g) if latent else None)
    dev = {k: (v.to(DEV) if v is not None else None) for k, v in w.items()}
    p = moe.pack_weights(dev, n_shared=ns)
    torch.cuda.synchronize()
    assert p["layout"] == moe.MOE_LAYOUT_FRAG16
    for k, v in w.items():
        if v is None:
            assert p[k] is None
            continue
        got = p[k].cpu().view(torch.int16)
        ref = frag16_reference(v).view(torch.int16)
        assert torch.equal(got, ref), k
        # and the sources are left as they were
        assert torch.equal(dev[k].cpu().view(torch.int16), v.view(torch.int16)), k


def test_pack_fp8_routed_experts():
    # FP8 routed matrices take the 16 x 64 byte blocks, the bf16 shared ones
    # the 16 x 32 element blocks; the block scales are handed back untouched
    log("[gpu] pack layout fp8")
    g = torch.Generator().manual_seed(4)
    E, F, d, ns, Fs = 3, 256, 384, 1, 64
    codes = lambda shape: torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)  # noqa: E731
    w = dict(W_gate=codes((E, F, d)), W_up=codes((E, F, d)), W_down=codes((E, d, F)),
             Ws_gate=_rand((ns * Fs, d), g), Ws_up=_rand((ns * Fs, d), g), Ws_down=_rand((d, ns * Fs), g))
    sc = dict(W_gate_scale=codes((E, F // 128, d // 128)), W_up_scale=codes((E, F // 128, d // 128)),
              W_down_scale=codes((E, d // 128, F // 128)))
    dev = {k: v.to(DEV) for k, v in w.items()}
    for k in ("W_gate", "W_up", "W_down"):
        dev[k] = dev[k].view(torch.float8_e4m3fn)
    dev.update({k: v.to(DEV) for k, v in sc.items()})
    p = moe.pack_weights(dev, n_shared=ns)
    torch.cuda.synchronize()
    for k in ("W_gate", "W_up", "W_down"):
        assert p[k].dtype == torch.float8_e4m3fn
        assert torch.equal(p[k].cpu().view(torch.uint8), frag16_fp8_reference(w[k])), k
    for k in ("Ws_gate", "Ws_up", "Ws_down"):
        assert torch.equal(p[k].cpu().view(torch.int16), frag16_reference(w[k]).view(torch.int16)), k
    for k in sc:
        assert p[k] is dev[k]
