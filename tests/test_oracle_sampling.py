"""Pins of the sampling-mode oracle (no GPU): Philox4x32-10 against its
published known-answer vectors, the uniform draws' distribution, the row
statistics against library routines, card sampling against the distribution
it samples, typical acceptance in its limits (greedy at low temperature,
everything at eps = 0), and the block policy's closed form."""
import math

import numpy as np
import pytest
from scipy import stats as sst
from scipy.special import softmax

from oracle import dflash as D
from oracle import sampling as S


def test_philox_known_answers():
    # known-answer vectors published with the Philox4x32-10 generator
    assert S.philox4x32_10([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert S.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert S.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_uniform_draws_are_uniform_and_distinct():
    u = np.array([S.uniform(20260829, r, q, i) for r in range(40) for q in range(5) for i in range(100)])
    assert np.all((u >= 0) & (u < 1))
    assert sst.kstest(u, "uniform").pvalue > 1e-3
    assert len(np.unique(u)) > 0.99 * len(u)
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))           # 24 bits


def test_row_stats_match_library_softmax_and_entropy():
    rng = np.random.default_rng(0)
    z = rng.standard_normal(5000).astype(np.float32) * 3
    for T in (1.0, 0.7, 2.0):
        p, H = S.row_stats(z, T)
        np.testing.assert_allclose(p, softmax(z.astype(np.float64) / T), rtol=1e-12, atol=0)
        assert H == pytest.approx(sst.entropy(softmax(z.astype(np.float64) / T)), rel=1e-12)


def test_card_sample_follows_the_kept_distribution():
    rng = np.random.default_rng(1)
    z = rng.standard_normal(300).astype(np.float32) * 2
    T, k, top_p = 0.8, 20, 0.9
    order = np.lexsort((np.arange(300), -z.astype(np.float64)))[:k]
    q = softmax(z[order].astype(np.float64) / T)
    keep = int(np.argmax(np.cumsum(q) >= top_p)) + 1
    target = q[:keep] / q[:keep].sum()
    N = 20000
    counts = {}
    for i in range(N):
        t = S.card_sample(z, T, k, top_p, (i + 0.5) / N)
        counts[t] = counts.get(t, 0) + 1
    assert set(counts) == set(order[:keep].tolist())
    for j in range(keep):
        assert abs(counts[int(order[j])] / N - target[j]) <= 2.0 / N
    # limits: top-k 1 or a tiny top-p is the argmax (lowest index on ties)
    zt = z.copy()
    zt[7] = zt[11] = zt.max() + 1
    for u in (0.0, 0.5, 0.999):
        assert S.card_sample(zt, T, 1, 1.0, u) == 7
        assert S.card_sample(zt, T, 20, 1e-9, u) == 7


def test_typical_accept_limits():
    rng = np.random.default_rng(2)
    B, V = 6, 50
    for trial in range(200):
        logits = rng.standard_normal((B, V)).astype(np.float32) * 4
        am = np.argmax(logits, 1)
        draft = [int(am[i]) if rng.random() < 0.7 else int((am[i] + 1) % V) for i in range(B - 1)]
        # low temperature: the target's distribution is its argmax, so typical acceptance is the greedy rule
        g = S.typical_accept(draft, logits, 1e-3, 0.2, None, 20, 0.95, 5, trial, 0)
        ref = D.accept(draft, am.tolist())
        assert (g["acc"], g["emitted"], g["n_emit"]) == (ref["acc"], ref["emitted"], ref["n_emit"])
        # eps = 0: every draft is accepted, the bonus comes from the last row
        a = S.typical_accept(draft, logits, 1.0, 0.0, 1.0, 20, 0.95, 5, trial, 1)
        assert a["acc"] == B - 1 and a["emitted"][:B - 1] == draft
        assert a["emitted"][-1] == S.card_sample(logits[B - 1], 1.0, 20, 0.95, S.uniform(5, trial, 1, B - 1))


def test_typical_accept_threshold_and_clamps():
    V = 8
    z = np.full((3, V), -10.0, dtype=np.float32)
    z[:, 3] = 0.0                      # p(3) close to 1, entropy close to 0
    z[1, 5] = z[1, 6] = 0.0            # row 1: tokens 3, 5 and 6 share the mass (p ~ 1/3, H ~ log 3)
    p1, H1 = S.row_stats(z[1], 1.0)
    thr = min(0.2, math.sqrt(0.2) * math.exp(-H1))
    assert p1[5] > thr                 # so 5 is accepted at row 1 with eps 0.2 (threshold ~ 0.149) ...
    r = S.typical_accept([3, 5], z, 1.0, 0.2, None, 20, 0.95, 1, 0, 0)
    assert r["acc"] == 2 and r["emitted"][:2] == [3, 5]
    r = S.typical_accept([3, 5], z, 1.0, 0.6, 1.2, 20, 0.95, 1, 0, 0)   # ... and rejected at threshold ~ 0.4
    assert p1[5] <= min(0.6, 1.2 * math.exp(-H1))
    assert r["acc"] == 1 and r["emitted"][0] == 3
    r = S.typical_accept([3, 5], z, 1.0, 0.2, None, 20, 0.95, 1, 0, 0, eos_id=5)
    assert r["emitted"] == [3, 5] and r["n_emit"] == 2
    r = S.typical_accept([3, 5], z, 1.0, 0.2, None, 20, 0.95, 1, 0, 0, budget=1)
    assert r["emitted"] == [3] and r["acc"] == 0


def test_block_policy_closed_form():
    p = S.BlockPolicy(8)
    assert p.next_block() == 8                       # m = 7 at the start
    for _ in range(20):
        p.update(0)
    assert p.next_block() == 2 and p.mean < 1e-5     # m halves each round
    p.update(7)                                      # m = 3.5 (+ a tiny rest) -> 4 -> 6
    assert p.next_block() == 6
    q = S.BlockPolicy(16)
    seq = [3, 3, 3, 3, 3, 3, 3, 3, 3, 3]
    for a in seq:
        q.update(a)
    m = 15.0
    for a in seq:
        m = 0.5 * m + 0.5 * a
    assert q.mean == m and q.next_block() == min(16, max(2, math.floor(m + 0.5) + 2))


def test_block_policy_degenerate_blocks():
    """Block 1 (target-only rounds) stays 1; block 2 stays 2 whatever is accepted."""
    p1, p2 = S.BlockPolicy(1), S.BlockPolicy(2)
    for a in (0, 0, 1, 0):
        assert p1.next_block() == 1 and p2.next_block() == 2
        p1.update(0)
        p2.update(a)
