"""CPU checks of the parity helpers themselves: the every-rank top-k check
passes for an exact top-k of logits within a known error of the oracle's, and
fails for a planted wrong id, a swapped pair of ranks and a repeated id."""
import numpy as np
import pytest

from tests import harness as Hn


def _case(seed=0, rows=6, V=5000, k=16, err=1e-3):
    rng = np.random.default_rng(seed)
    L = rng.normal(size=(rows, V))
    G = L + rng.uniform(-err, err, size=L.shape)
    ids = np.stack([np.lexsort((np.arange(V), -G[r]))[:k] for r in range(rows)]).astype(np.int32)
    return L, G, ids, k


def test_exact_topk_within_error_passes():
    L, G, ids, k = _case()
    assert Hn.topk_valid_within_error(L, ids, k, G) == L.shape[0] * k
    comp, excl = Hn.topk_agrees_away_from_ties(L, ids, k, gpu_logits=G)
    assert comp + excl == L.shape[0] * k


def test_planted_wrong_id_fails():
    L, G, ids, k = _case(seed=1)
    bad = ids.copy()
    bad[2, 5] = int(np.argmin(L[2]))   # the row's smallest logit
    with pytest.raises(AssertionError):
        Hn.topk_valid_within_error(L, bad, k, G)


def test_planted_rank_swap_fails():
    L, G, ids, k = _case(seed=2)
    bad = ids.copy()
    bad[1, [0, k - 1]] = bad[1, [k - 1, 0]]   # the largest and the k-th swapped
    with pytest.raises(AssertionError):
        Hn.topk_valid_within_error(L, bad, k, G)


def test_repeated_id_fails():
    L, G, ids, k = _case(seed=3)
    bad = ids.copy()
    bad[0, 3] = bad[0, 2]
    with pytest.raises(AssertionError):
        Hn.topk_valid_within_error(L, bad, k, G)
