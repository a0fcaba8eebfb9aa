"""Pins of the oracle's first-mismatch accept rule (no GPU)."""
import itertools

import pytest

from oracle import dflash as D


def _characterize(draft, verify, res):
    """What any correct first-mismatch accept must satisfy (no EOS, no budget):
    the emitted tokens are the longest matching draft prefix followed by the
    verify token at the first mismatch (or the bonus token when all match)."""
    n = res["n_emit"]
    em = res["emitted"]
    assert 1 <= n <= len(draft) + 1 and len(em) == n
    assert em[:-1] == list(draft[: n - 1])
    assert all(draft[j] == verify[j] for j in range(n - 1))
    if n - 1 < len(draft):
        assert draft[n - 1] != verify[n - 1]
    assert em[-1] == verify[n - 1]
    assert res["acc"] == n - 1


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_accept_exhaustive_small_vocab(B):
    V = 3
    count = 0
    for draft in itertools.product(range(V), repeat=B - 1):
        for verify in itertools.product(range(V), repeat=B):
            _characterize(draft, verify, D.accept(draft, verify))
            count += 1
    assert count == V ** (2 * B - 1)


def test_accept_named_cases():
    # first-token rejection: emit exactly the target's token
    r = D.accept([5, 6, 7], [9, 6, 7, 8])
    assert r == {"acc": 0, "emitted": [9], "n_emit": 1}
    # full acceptance plus the bonus token
    r = D.accept([5, 6, 7], [5, 6, 7, 8])
    assert r == {"acc": 3, "emitted": [5, 6, 7, 8], "n_emit": 4}
    # EOS inside the accepted run: keep up to and including the first EOS
    r = D.accept([5, 2, 7], [5, 2, 7, 8], eos_id=2)
    assert r == {"acc": 1, "emitted": [5, 2], "n_emit": 2}
    # EOS as the bonus / correction token
    r = D.accept([5, 6, 7], [5, 2, 1, 1], eos_id=2)
    assert r == {"acc": 1, "emitted": [5, 2], "n_emit": 2}
    # remaining budget smaller than the block
    r = D.accept([5, 6, 7], [5, 6, 7, 8], budget=2)
    assert r == {"acc": 1, "emitted": [5, 6], "n_emit": 2}
    r = D.accept([5, 6, 7], [5, 6, 7, 8], budget=0)     # a verified round emits at least 1
    assert r["n_emit"] == 1 and r["emitted"] == [5]
    # block size 1: no draft rows, a plain target step
    r = D.accept([], [42])
    assert r == {"acc": 0, "emitted": [42], "n_emit": 1}


def test_next_block():
    assert D.next_block([3, 4, 9], 4, 99) == [9, 99, 99, 99]
    assert D.next_block([3], 1, 99) == [3]
