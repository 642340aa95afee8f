"""Host logic of the parity checks (no GPU): the full-size token sample
covers every tile it promises, and the output check fails on a mistake
confined to one element or one token even when the aggregate error would
pass."""
import numpy as np
import pytest

import oracle
from parity import (RANDOM_LAYER_SEEDS, RANDOM_ROUTER_SEEDS, RESULTS, TIE, check_output,
                    coverage_tokens, random_layer, random_router)


def _routing(T, E, K, seed, skew=0.5):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)) + skew * (rng.permutation(E) + 1.0) ** -1.1
    idx = np.sort(np.argsort(-logits, 1)[:, :K], 1).astype(np.int32)
    return idx, oracle.dispatch(idx, E)


@pytest.mark.parametrize("T,E,K,bm,seed", [(16384, 384, 8, 128, 1), (4096, 896, 16, 128, 2),
                                           (3000, 40, 3, 128, 3), (700, 6, 2, 128, 4)])
def test_coverage_sample_hits_every_tile(T, E, K, bm, seed):
    idx, d = _routing(T, E, K, seed)
    gap = np.ones(T)
    gap[[5, 17]] = 1e-7                       # two near-tie tokens
    toks = coverage_tokens(T, K, d["counts"], d["offsets"], d["sorted_token"], idx, gap, bm=bm,
                           n_random=64)
    mask = np.zeros(T, bool)
    mask[toks] = True
    assert mask[5] and mask[17] and mask[T - 1]
    st = d["sorted_token"]
    for e in range(E):
        lo, hi = d["offsets"][e], d["offsets"][e + 1]
        if hi == lo:
            continue
        for c in range(lo, hi, bm):           # every M tile of the expert
            assert mask[st[c:min(c + bm, hi)]].any(), (e, c)
        assert mask[st[hi - 1]], e            # its ragged last row
    for c in range(0, T, bm):                 # every shared-expert tile
        assert mask[c:c + bm].any(), c
    assert len(toks) < T


def test_check_output_catches_local_mistakes():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((64, 1024))
    noise = ref * (1 + rng.uniform(-2 ** -9, 2 ** -9, ref.shape)) + 2e-3 * rng.standard_normal(ref.shape)
    n0 = len(RESULTS)
    rec = check_output("clean", noise, ref, "bf16", False)
    assert rec["rel_l2"] < 5e-3 and rec["elem_ratio"] < 1
    one = noise.copy()
    one[7, 100] += 0.5                        # one wrong element: aggregate L2 still passes
    with pytest.raises(AssertionError, match="element"):
        check_output("one element", one, ref, "bf16", False)
    block = noise.copy()
    block[3, 16:32] = rng.standard_normal(16) * 0.2   # one 16-column block of one token
    with pytest.raises(AssertionError):
        check_output("one block", block, ref, "bf16", False)
    tok = noise.copy()
    tok[9] *= 1.05                            # one token off by 5%: only the per-token bound fails
    assert np.linalg.norm(tok - ref) / np.linalg.norm(ref) < 2e-2
    with pytest.raises(AssertionError, match="tokens above"):
        check_output("one token", tok, ref, "bf16", False)
    # tokens whose reference is exactly zero (an expert-parallel slice with
    # none of its experts): an exact zero passes, anything else fails
    zref, zgot = ref.copy(), noise.copy()
    zref[5] = 0.0
    zgot[5] = 0.0
    assert check_output("zero token", zgot, zref, "bf16", False)["elem_ratio"] < 1
    zgot[5, 3] = 1e-30
    with pytest.raises(AssertionError):
        check_output("zero token, one tiny element", zgot, zref, "bf16", False)
    del RESULTS[n0:]


def test_tie_threshold_is_the_stated_one():
    assert TIE == 1e-5


def test_random_layers_span_the_tile_regimes():
    # The seeded random layers of the GPU parity test fall on both sides of
    # each batch-size switch: 16-row and 128-row expert tiles (below and from
    # 10 rows per expert on average) for bf16 rows, packed bf16 and FP8;
    # single tokens; latent layers below and from 512 tokens; hot experts;
    # no and eight shared experts; fp32 and bf16 activations.  All within
    # the ABI's limits.
    draws = [random_layer(s) for s in RANDOM_LAYER_SEEDS]

    def has(pred):
        return any(pred(kw, packed, hot) for kw, packed, hot in draws)

    def rows(kw):
        return kw["T"] * kw["K"] / kw["E"]

    for w, pk in (("bf16", False), ("bf16", True), ("fp8", True)):
        assert has(lambda kw, p, h: kw["w_dtype"] == w and p == pk and rows(kw) >= 10), (w, pk)
        assert has(lambda kw, p, h: kw["w_dtype"] == w and p == pk and rows(kw) < 10), (w, pk)
    assert has(lambda kw, p, h: kw["T"] == 1)
    assert has(lambda kw, p, h: kw["d_latent"] > 0 and kw["T"] >= 512)
    assert has(lambda kw, p, h: kw["d_latent"] > 0 and kw["T"] < 512)
    assert has(lambda kw, p, h: h is not None)
    assert has(lambda kw, p, h: kw["n_shared"] == 0) and has(lambda kw, p, h: kw["n_shared"] == 8)
    assert {kw["act_dtype"] for kw, _, _ in draws} == {"bf16", "f32"}
    for kw, packed, hot in draws:
        assert 1 <= kw["K"] <= min(kw["E"], 16) and kw["E"] <= 1024 and kw["T"] >= 1
        assert kw["d"] % 64 == 0 and kw["F"] % 64 == 0 and kw["d_latent"] % 64 == 0
        assert kw["n_shared"] <= 8 and kw["F_shared"] % 64 == 0
        if kw["w_dtype"] == "fp8":
            assert packed and (kw["d_latent"] or kw["d"]) % 128 == 0 and kw["F"] % 128 == 0
        assert hot is None or 0 <= hot < kw["E"]


def test_random_routers_span_the_regimes():
    # The seeded random router shapes: both logit tile forms (up to 64
    # tokens and above), one and several split-K planes, fp32 and bf16,
    # flat and group-limited choice, groups kept with fewer experts than K
    # (the masked scores are chosen), one expert; all within the ABI.
    draws = [random_router(s) for s in RANDOM_ROUTER_SEEDS]
    assert any(kw["T"] <= 64 for kw, _, _ in draws) and any(kw["T"] > 4096 for kw, _, _ in draws)
    assert {kw["act_dtype"] for kw, _, _ in draws} == {"bf16", "f32"}
    assert any(g > 1 for _, g, _ in draws) and any(g == 1 for _, g, _ in draws)
    assert any(g > 1 and kw["K"] > tg * (kw["E"] // g) for kw, g, tg in draws)
    assert any(kw["E"] == 1 for kw, _, _ in draws) and any(kw["E"] == 1024 for kw, _, _ in draws)
    for kw, g, tg in draws:
        assert 1 <= kw["K"] <= min(kw["E"], 16) and kw["E"] <= 1024 and kw["d"] % 64 == 0
        if g > 1:
            assert g <= 64 and kw["E"] % g == 0 and kw["E"] // g >= 2 and 1 <= tg <= g
