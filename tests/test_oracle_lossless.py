"""Losslessness of the speculative loop with the oracle drafter and the tiny
synthetic target (no GPU): output must equal greedy decoding token for token."""
import numpy as np
import pytest

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from oracle import target as T


def _np(w):
    return {k: ([synth.bf16_to_f32_numpy(t) for t in v] if isinstance(v, list) else synth.bf16_to_f32_numpy(v))
            for k, v in w.items()}


@pytest.fixture(scope="module")
def setup():
    cfg = config.tiny()
    Wd = _np(synth.make_weights(cfg, seed=0))
    tcfg = cfg.replace(n_layers=2)
    Wt = _np(synth.make_weights(tcfg, seed=11))
    Wt["embed"], Wt["lm_head"] = Wd["embed"], Wd["lm_head"]      # shared with the drafter
    Wt["embed"] = Wt["embed"] * 30.0   # a peakier target so greedy continuations vary
    Wd["embed"] = Wt["embed"]
    tgt = T.TinyTarget(tcfg, Wt, n_layers=2)
    return cfg, Wd, tgt


def test_greedy_is_deterministic_and_batch_invariant(setup):
    cfg, Wd, tgt = setup
    prompt = [5, 17, 300, 4000, 12]
    g1 = T.greedy(tgt, prompt, 20)
    # feeding the greedy continuation as one verify block gives the same argmaxes
    tgt.reset()
    ids, _ = tgt.feed(prompt + g1[:-1], 0)
    assert ids[len(prompt) - 1:] == g1
    assert T.greedy(tgt, prompt, 20) == g1


def test_lossless_with_oracle_drafter(setup):
    cfg, Wd, tgt = setup
    prompt = [5, 17, 300, 4000, 12, 99]
    ref = T.greedy(tgt, prompt, 24)
    res = T.speculative(tgt, T.oracle_draft_fn(cfg, Wd), prompt, 24, cfg.block, cfg.window, cfg.mask_id)
    assert res["tokens"] == ref
    assert len(ref) == 24


@pytest.mark.parametrize("block", [1, 2, 8])
def test_lossless_with_planted_drafts(setup, block):
    """Drafts equal to the true continuation corrupted at a geometric position
    exercise long accepts, the bonus token and budget clamping."""
    cfg, Wd, tgt = setup
    prompt = [7, 8, 9, 1000]
    n_new = 37
    ref = T.greedy(tgt, prompt, n_new + block)
    rng = np.random.default_rng(block)

    def planted(blk, pos, vf, taps):
        start = pos - len(prompt) + 1          # index in ref of the token after blk[0]
        d = list(ref[start:start + block - 1])
        d += [0] * (block - 1 - len(d))
        a = min(int(rng.geometric(0.3)) - 1, block - 1)
        if a < block - 1:
            d[a] = (d[a] + 1) % cfg.vocab
        return d

    res = T.speculative(tgt, planted, prompt, n_new, block, cfg.window, cfg.mask_id)
    assert res["tokens"] == ref[:n_new]
    if block > 1:
        assert max(res["accepts"]) >= min(2, block - 1)


def test_lossless_stops_at_eos(setup):
    cfg, Wd, tgt = setup
    prompt = [5, 17, 300, 4000, 12, 99]
    full = T.greedy(tgt, prompt, 30)
    eos = full[9]
    ref = T.greedy(tgt, prompt, 30, eos_id=eos)
    assert ref[-1] == eos and len(ref) <= 10

    def planted(blk, pos, vf, taps):
        start = pos - len(prompt) + 1
        d = list(full[start:start + cfg.block - 1])
        return d + [0] * (cfg.block - 1 - len(d))

    res = T.speculative(tgt, planted, prompt, 30, cfg.block, cfg.window, cfg.mask_id, eos_id=eos)
    assert res["tokens"] == ref


def test_block_one_is_plain_greedy(setup):
    cfg, Wd, tgt = setup
    prompt = [3, 4]
    ref = T.greedy(tgt, prompt, 12)
    res = T.speculative(tgt, lambda *a: [], prompt, 12, 1, cfg.window, cfg.mask_id)
    assert res["tokens"] == ref and all(a == 0 for a in res["accepts"])


def test_block_len_cases():
    # the configured block while budget and capacity are large
    assert D.block_len(8, 100, 10, 1000, 50) == 8
    # the budget binds: 3 tokens left -> a block of 3 (2 drafts + the target's token)
    assert D.block_len(8, 100, 97, 1000, 50) == 3
    # the sequence capacity binds
    assert D.block_len(8, 100, 10, 55, 50) == 5
    # one token left: a target-only step
    assert D.block_len(16, 24, 23, 1000, 7) == 1
    # nothing left
    assert D.block_len(8, 24, 24, 1000, 7) <= 0 and D.block_len(8, 100, 10, 50, 50) <= 0


@pytest.mark.parametrize("max_seq_extra", [None, 19])
def test_lossless_with_dynamic_block_len(setup, max_seq_extra):
    """Rounds shrink at the end of the budget (and of the sequence capacity):
    the output is still the target's greedy decoding, ends exactly at the budget
    (or where the capacity stops it), and no round runs past either bound."""
    cfg, Wd, tgt = setup
    prompt = [5, 17, 300, 4000, 12, 99]
    n_new = 23
    max_seq = None if max_seq_extra is None else len(prompt) + max_seq_extra
    res = T.speculative(tgt, T.oracle_draft_fn(cfg, Wd), prompt, n_new, cfg.block, cfg.window, cfg.mask_id,
                        dynamic=True, max_seq=max_seq)
    n_expect = n_new if max_seq is None else min(n_new, max_seq - len(prompt) + 1)
    assert res["tokens"] == T.greedy(tgt, prompt, n_expect)
    assert all(1 <= b <= cfg.block for b in res["blocks"])
    fed = len(prompt) + len(res["tokens"]) - 1   # positions fed to the target: all but the last token
    assert max_seq is None or fed <= max_seq
    assert res["blocks"][-1] < cfg.block    # the last round was shrunk


def test_target_mirror_mode_drift_is_small(setup):
    """The mirror target (bf16 at the drafter's cast points) stays close to the
    exact one and agrees on the argmax of every row of a short feed."""
    cfg, Wd, tgt = setup
    Wt = {k: getattr(tgt, "W")[k] for k in tgt.W}
    mir = T.TinyTarget(tgt.cfg, Wt, n_layers=2, mode="mirror")
    toks = [5, 17, 300, 4000, 12, 99, 7, 8]
    tgt.reset()
    ids_e, taps_e, lg_e = tgt.feed(toks, 0, want_logits=True)
    ids_m, taps_m, lg_m = mir.feed(toks, 0, want_logits=True)
    drift = np.max(np.abs(lg_m - lg_e)) / np.max(np.abs(lg_e))
    assert 0 < drift < 0.05
    assert ids_m == ids_e
    for a, b in zip(taps_e, taps_m):
        assert np.max(np.abs(a - b)) <= 0.05 * np.max(np.abs(a))


@pytest.mark.parametrize("mode", ["exact", "mirror"])
def test_target_prefill_equals_feed(setup, mode):
    """The batched prefix routine leaves the same cache as feeding the prompt row
    by row: the rows fed afterwards get the same logits and taps."""
    cfg, Wd, tgt = setup
    Wt = {k: tgt.W[k] for k in tgt.W}
    a = T.TinyTarget(tgt.cfg, Wt, n_layers=2, mode=mode)
    b = T.TinyTarget(tgt.cfg, Wt, n_layers=2, mode=mode)
    prompt = [5, 17, 300, 4000, 12, 99, 7, 8, 1, 2, 3, 4, 5]
    nxt = [44, 45, 46]
    a.feed(prompt, 0)
    _, ta, la = a.feed(nxt, len(prompt), want_logits=True)
    b.prefill(prompt[:6])
    b.prefill(prompt[6:])
    assert b.length == len(prompt)
    _, tb, lb = b.feed(nxt, len(prompt), want_logits=True)
    # exact: fp64 summation order only; mirror: a bf16 rounding may flip at a tie
    tol = 1e-10 if mode == "exact" else 1e-3
    assert np.max(np.abs(la - lb)) <= tol * np.max(np.abs(la))
    for x, y in zip(ta, tb):
        assert np.max(np.abs(x - y)) <= max(tol, 1e-6) * np.max(np.abs(x))
    for l in range(2):
        assert np.max(np.abs(a.k[l] - b.k[l])) <= tol * np.max(np.abs(a.k[l]))
