"""Host logic of the parity checks (no GPU): the full-size token sample
covers every tile it promises, and the output check fails on a mistake
confined to one element or one token even when the aggregate error would
pass."""
import numpy as np
import pytest

import oracle
from parity import RESULTS, TIE, check_output, coverage_tokens


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
    del RESULTS[n0:]


def test_tie_threshold_is_the_stated_one():
    assert TIE == 1e-5
