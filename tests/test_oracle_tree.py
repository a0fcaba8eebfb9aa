"""Pins of the candidate-tree oracle (no GPU): the selection rule against a
brute-force global sort, the list log-probabilities against a library
log-softmax, tree acceptance against an independent formulation and against
the chain rule, and the lossless tree loop against greedy decoding."""
import itertools

import numpy as np
import pytest
from scipy.special import log_softmax

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from oracle import target as T
from oracle import tree as TR


def _lists(rng, Dm, k, V=1000):
    ids = np.stack([rng.choice(V, size=k, replace=False) for _ in range(Dm)])
    vals = -np.sort(-rng.standard_normal((Dm, k)).astype(np.float32), axis=1)
    return ids, vals


def test_list_logprobs_are_the_softmax_of_the_list():
    rng = np.random.default_rng(0)
    _, vals = _lists(rng, 5, 16)
    lp = TR.list_logprobs(vals)
    np.testing.assert_allclose(lp, log_softmax(vals.astype(np.float64), axis=1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.exp(lp).sum(1), 1.0, atol=1e-13)
    assert np.all(np.diff(lp, axis=1) <= 0)


def _brute_tree(root, ids, vals, n):
    """Every node up to depth B-1 scored independently, the chain first, then the
    rest by (score desc, depth asc, rank path lexicographic asc)."""
    Dm, k = ids.shape
    lp = log_softmax(vals.astype(np.float64), axis=1)
    chain = [tuple([0] * d) for d in range(1, Dm + 1)][: max(0, n - 1)]
    nodes = []
    for d in range(1, Dm + 1):
        for path in itertools.product(range(k), repeat=d):
            if path in chain:
                continue
            nodes.append((-sum(lp[e][path[e]] for e in range(d)), d, path))
    nodes.sort()
    order = chain + [p for _, _, p in nodes][: max(0, n - 1 - len(chain))]
    return [root] + [int(ids[len(p) - 1][p[-1]]) for p in order], order


@pytest.mark.parametrize("seed", range(6))
def test_build_tree_matches_a_brute_force_global_sort(seed):
    rng = np.random.default_rng(seed)
    Dm, k = 4, 3
    ids, vals = _lists(rng, Dm, k)
    for n in (1, 2, 4, 5, 9, 17, 40, 121):
        t = TR.build_tree(7, ids, vals, n)
        toks, order = _brute_tree(7, ids, vals, n)
        assert t["tokens"] == toks, (seed, n)
        # the rank path of every node, from the parent links
        paths = [tuple(t["rank"][j] for j in TR.root_path(t["parent"], i)[1:]) for i in range(1, len(t["tokens"]))]
        assert paths == order
        assert len(t["tokens"]) == min(n, 1 + sum(k ** d for d in range(1, Dm + 1)))
        for i in range(1, len(t["tokens"])):
            assert t["parent"][i] < i and t["depth"][i] == t["depth"][t["parent"][i]] + 1


def test_build_tree_tie_breaks():
    # equal values everywhere: every candidate has the same log-probability, so
    # after the chain the order is depth first, then parent index, then rank
    ids = np.array([[10, 11, 12], [20, 21, 22], [30, 31, 32]])
    vals = np.zeros((3, 3), dtype=np.float32)
    t = TR.build_tree(1, ids, vals, 9)
    assert t["tokens"] == [1, 10, 20, 30, 11, 12, 21, 22, 20]
    assert t["parent"] == [-1, 0, 1, 2, 0, 0, 1, 1, 4]
    assert t["rank"] == [-1, 0, 0, 0, 1, 2, 1, 2, 0]


def _brute_accept(tokens, parent, verify):
    """The deepest node whose every edge (u -> v) on its root path has
    tokens[v] == verify[u]."""
    best = 0
    for i in range(len(tokens)):
        path = TR.root_path(parent, i)
        if all(tokens[v] == verify[u] for u, v in zip(path, path[1:])):
            if len(path) > len(TR.root_path(parent, best)):
                best = i
    return best


def test_tree_accept_exhaustive_tiny_vocab():
    """Every verify vector over a 3-token vocabulary, on every tree of up to 6
    nodes built from 2-candidate lists: the walk ends at the deepest consistent
    node, and emits that path plus the target's token there."""
    rng = np.random.default_rng(3)
    V, Dm, k = 3, 3, 2
    checked = 0
    for _ in range(4):
        ids = np.stack([rng.permutation(V)[:k] for _ in range(Dm)])
        vals = -np.sort(-rng.standard_normal((Dm, k)).astype(np.float32), axis=1)
        for n in range(1, 7):
            t = TR.build_tree(int(rng.integers(V)), ids, vals, n)
            for verify in itertools.product(range(V), repeat=len(t["tokens"])):
                res = TR.tree_accept(t["tokens"], t["parent"], list(verify), Dm + 1)
                end = _brute_accept(t["tokens"], t["parent"], verify)
                path = TR.root_path(t["parent"], end)
                assert res["path"] == path and res["acc"] == len(path) - 1
                assert res["emitted"] == [t["tokens"][i] for i in path[1:]] + [verify[end]]
                checked += 1
    assert checked > 1000


def test_tree_accept_on_a_chain_is_the_chain_rule():
    rng = np.random.default_rng(4)
    B = 5
    for _ in range(300):
        d = rng.integers(0, 3, B - 1).tolist()
        v = rng.integers(0, 3, B).tolist()
        eos = int(rng.integers(-1, 3))
        budget = int(rng.integers(1, B + 2)) if rng.random() < 0.5 else None
        tokens = [int(rng.integers(0, 3))] + d
        parent = list(range(-1, B - 1))
        a = TR.tree_accept(tokens, parent, v, B, eos_id=eos, budget=budget)
        b = D.accept(d, v, eos_id=eos, budget=budget)
        assert (a["acc"], a["emitted"], a["n_emit"]) == (b["acc"], b["emitted"], b["n_emit"])
        assert a["path"] == list(range(b["n_emit"]))


def test_tree_accept_is_at_least_the_chain_accept():
    """The tree contains the top-1 chain, so on the same lists and the same
    target it never accepts less; with the target's token often at rank > 0 it
    accepts more."""
    rng = np.random.default_rng(5)
    Dm, k, n = 7, 16, 24
    gain = 0
    for _ in range(400):
        ids, vals = _lists(rng, Dm, k)
        # the target's continuation: rank 0 w.p. 0.6, another listed rank w.p. 0.3, unlisted otherwise
        g = []
        for d in range(Dm):
            u = rng.random()
            g.append(int(ids[d][0]) if u < 0.6 else int(ids[d][rng.integers(1, k)]) if u < 0.9 else 5000 + d)
        t = TR.build_tree(1, ids, vals, n)
        verify = [g[t["depth"][i]] if t["depth"][i] < Dm else 0 for i in range(len(t["tokens"]))]
        a_tree = TR.tree_accept(t["tokens"], t["parent"], verify, Dm + 1)["acc"]
        a_chain = D.accept([int(x) for x in ids[:, 0]], g + [0])["acc"]
        assert a_tree >= a_chain
        gain += a_tree - a_chain
    assert gain > 0


@pytest.fixture(scope="module")
def tiny_pair():
    cfg = config.tiny()

    def np_(w):
        return {kk: ([synth.bf16_to_f32_numpy(t) for t in v] if isinstance(v, list) else synth.bf16_to_f32_numpy(v))
                for kk, v in w.items()}
    Wd = np_(synth.make_weights(cfg, seed=0))
    tcfg = cfg.replace(n_layers=2)
    Wt = np_(synth.make_weights(tcfg, seed=11))
    Wt["embed"] = Wd["embed"] * 30.0
    Wt["lm_head"] = Wd["lm_head"]
    Wd["embed"] = Wt["embed"]
    return cfg, Wd, T.TinyTarget(tcfg, Wt, n_layers=2)


def test_tree_verify_of_a_chain_equals_a_block_feed(tiny_pair):
    cfg, _, tgt = tiny_pair
    prompt = [5, 17, 300, 4000]
    tgt.reset()
    tgt.feed(prompt, 0)
    blk = [12, 99, 7, 8]
    verify, taps = TR.tree_verify(tgt, blk, [-1, 0, 1, 2], len(prompt))
    assert tgt.length == len(prompt)
    ids, ftaps = tgt.feed(blk, len(prompt))
    assert verify == ids
    for a, b in zip(taps, ftaps):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("mode", ["drafter", "planted"])
def test_tree_loop_is_lossless(tiny_pair, mode):
    """The tree round loop emits exactly the target's greedy continuation, with
    the oracle drafter's top-16 lists and with planted lists that hold the true
    continuation at a random rank (where the tree accepts more than the chain)."""
    cfg, Wd, tgt = tiny_pair
    prompt = [5, 17, 300, 4000, 12, 99]
    n_new, n_nodes = 30, 16
    ref = T.greedy(tgt, prompt, n_new + cfg.block)
    rng = np.random.default_rng(7)

    def drafter(blk, pos, taps):
        lg = D.draft_block(cfg, Wd, taps, blk, pos, 0, "mirror")["logits"]
        return D.topk(lg, 16)

    def planted(blk, pos, taps):
        start = pos - len(prompt) + 1
        ids = rng.permuted(np.tile(np.arange(cfg.vocab - 1), (cfg.block - 1, 1)), axis=1)[:, :16]
        for d in range(cfg.block - 1):
            true = ref[start + d] if start + d < len(ref) else 0
            ids[d] = [x if x != true else (x + 1) % (cfg.vocab - 1) for x in ids[d]]
            r = int(rng.integers(0, 4))
            if r < 3:
                ids[d][r] = true
        vals = -np.sort(-rng.standard_normal((cfg.block - 1, 16)).astype(np.float32), axis=1)
        return ids, vals

    res = TR.speculative_tree(tgt, drafter if mode == "drafter" else planted, prompt, n_new, cfg.block, n_nodes,
                              cfg.mask_id)
    assert res["tokens"][:n_new] == ref[:n_new] and len(res["tokens"]) == n_new
    if mode == "planted":
        assert max(res["accepts"]) >= 2
