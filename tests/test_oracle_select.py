"""Pins for the oracle's selection step.

Top-k: "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm", section
"The Prediction Problem" (the k best scores form the active set).  Ties go to the lower index
and the set is listed in ascending order (the reading taken here; the pages are silent).
Threshold: "Activation sparsity", section "Implementation sketch" (scores >= threshold).
"""
import itertools

import numpy as np
import pytest

from oracle import oracle as orc


def _dominates(s, A):
    """A is a valid top-|A| set under (score desc, index asc): every member outranks every
    non-member."""
    inside = set(A)
    for i in A:
        for j in range(len(s)):
            if j in inside:
                continue
            if not (s[i] > s[j] or (s[i] == s[j] and i < j)):
                return False
    return True


@pytest.mark.parametrize("f", range(0, 7))
def test_brute_force_every_tie_pattern(f):
    alphabet = [np.float32(0.25), np.float32(0.5), np.float32(0.75)]
    for pattern in itertools.product(alphabet, repeat=f):
        s = np.array(pattern, np.float32)
        for k in range(f + 1):
            valid = [A for A in itertools.combinations(range(f), k) if _dominates(s, A)]
            assert len(valid) == 1, (pattern, k, valid)
            assert orc.select_topk(s, k).tolist() == list(valid[0])


@pytest.mark.parametrize("seed", range(4))
def test_matches_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    f = 1500
    s = (np.round(rng.random(f) * 40) / 40).astype(np.float32)   # many ties
    for k in (0, 1, 7, 150, 749, 1499, 1500):
        ref = sorted(np.argsort(-s, kind="stable")[:k].tolist())
        assert orc.select_topk(s, k).tolist() == ref


def test_special_cases():
    s = np.array([0.3, 0.9, 0.1, 0.9, 0.5], np.float32)
    assert orc.select_topk(s, 0).tolist() == []
    assert orc.select_topk(s, 5).tolist() == [0, 1, 2, 3, 4]
    assert orc.select_topk(s, 1).tolist() == [1]                 # tie at 0.9: lower index
    assert orc.select_topk(np.full(9, 0.5, np.float32), 4).tolist() == [0, 1, 2, 3]
    # -0.0 and +0.0 are equal scores: the lower index wins either way round
    assert orc.select_topk(np.array([-0.0, 0.0, -1.0], np.float32), 1).tolist() == [0]
    assert orc.select_topk(np.array([0.0, -0.0, -1.0], np.float32), 1).tolist() == [0]
    # saturated sigmoid scores tie at 1.0
    assert orc.select_topk(np.array([0.2, 1.0, 1.0, 1.0], np.float32), 2).tolist() == [1, 2]


def test_topk_rejects_bad_k_and_non_finite():
    s = np.array([0.1, 0.2], np.float32)
    for k in (-1, 3):
        with pytest.raises(ValueError):
            orc.select_topk(s, k)
    with pytest.raises(ValueError):
        orc.select_topk(np.array([0.1, np.nan], np.float32), 1)


def test_threshold_special_cases_and_numpy():
    s = np.array([0.5, 0.49999997, 0.7, 0.5, 0.1], np.float32)
    assert orc.select_threshold(s, 0.5).tolist() == [0, 2, 3]    # equality is included
    assert orc.select_threshold(s, float(s.min())).tolist() == [0, 1, 2, 3, 4]
    assert orc.select_threshold(s, 0.70000005).tolist() == []
    assert orc.select_threshold(np.array([-0.0, 0.0], np.float32), 0.0).tolist() == [0, 1]
    rng = np.random.default_rng(5)
    s = rng.random(3000).astype(np.float32)
    for tau in (0.0, 0.25, 0.5, 0.999, 1.0):
        assert orc.select_threshold(s, tau).tolist() == np.nonzero(s >= np.float32(tau))[0].tolist()
