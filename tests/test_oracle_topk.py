"""Pins of the oracle's top-K (brute-force sort, ties, short contexts, torch.topk)."""
import numpy as np
import pytest
import torch

import oracle


def _brute(scores, K):
    order = sorted(range(len(scores)), key=lambda t: (-scores[t], t))
    sel = sorted(order[:K])
    return sel + [-1] * (K - len(sel))


@pytest.mark.parametrize("L", [1, 5, 16, 17, 40, 129])
@pytest.mark.parametrize("K", [1, 4, 16])
def test_matches_full_stable_sort_with_ties(L, K):
    rng = np.random.default_rng(L * 100 + K)
    scores = rng.integers(0, 6, L).astype(np.float64)          # many exact ties
    assert list(oracle.topk_select(scores, K)) == _brute(list(scores), K)


def test_short_context_selects_everything():
    out = oracle.topk_select(np.array([3.0, 1.0, 2.0]), 8)
    assert list(out) == [0, 1, 2, -1, -1, -1, -1, -1]


def test_all_equal_picks_lowest_indices():
    assert list(oracle.topk_select(np.zeros(100), 5)) == [0, 1, 2, 3, 4]


def test_duplicated_keys_tie_break_to_lower_index():
    s = np.array([1.0, 5.0, 2.0, 5.0, 5.0, 0.0])
    assert list(oracle.topk_select(s, 2)) == [1, 3]


def test_distinct_values_agree_with_torch_topk():
    rng = np.random.default_rng(9)
    s = rng.permutation(5000).astype(np.float64) * 0.37
    ref = torch.topk(torch.from_numpy(s), 2048).indices.numpy()
    assert np.array_equal(oracle.topk_select(s, 2048), np.sort(ref))


def test_output_is_ascending_and_padded():
    rng = np.random.default_rng(10)
    out = oracle.topk_select(rng.random(1000), 64)
    assert np.all(np.diff(out) > 0)
