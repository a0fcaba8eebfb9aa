"""The oracle against scalar brute force (no GPU).

``tests/brute.py`` restates the drafter round and the tiny causal target with
explicit loops and its own bf16 rounding. Agreement to fp64 rounding level pins:
  * every step of the drafter (hc mean, tap concat, fc, optional ctx RMSNorm,
    context K/V, bidirectional block attention, MLP, final norm, the LM head's
    row selection: rows 1..B-1);
  * the placement of every bf16 cast point of mirror mode: a cast dropped,
    added or moved changes values by about 2**-9 relative, far above the
    1e-10 bound used here;
  * the tiny target's per-row causal forward (positions, q/k gains, causal
    key range, taps after each layer).
"""
import struct

import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from oracle import target as T
from tests import brute


def _f64_weights(cfg, seed, embed_scale=20.0, mlp_scale=10.0):
    w = synth.make_weights(cfg, seed=seed)
    out = {k: ([synth.bf16_to_f32_numpy(t).astype(np.float64) for t in v] if isinstance(v, list)
               else synth.bf16_to_f32_numpy(v).astype(np.float64)) for k, v in w.items()}
    out["embed"] = out["embed"] * embed_scale   # a residual stream large enough to matter
    # at these tiny widths N(0, 0.02) projections would make the MLP's update a
    # rounding-level change of the residual; scaled up, every sublayer matters
    for name in ("wgu", "wd", "wo"):
        out[name] = [t * mlp_scale for t in out[name]]
    return out


def _small(**kw):
    return config.tiny(block=3, window=5).replace(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48,
                                                  vocab=64, tap_hidden=32, mask_id=63, **kw)


def test_bf16_rne_against_torch_and_bit_patterns():
    # fp32 inputs: torch's fp32 -> bf16 conversion rounds once, to nearest even
    g = torch.Generator().manual_seed(0)
    x = torch.randn(20000, generator=g) * torch.exp2(torch.randint(-60, 60, (20000,), generator=g).float())
    ref = x.to(torch.bfloat16).float().double().numpy()
    got = np.array([brute.bf16_rne(v) for v in x.double().numpy()])
    np.testing.assert_array_equal(got, ref)
    # halfway cases, built from bit patterns: 1 + 2**-8 is a tie between 1 and 1 + 2**-7
    assert brute.bf16_rne(1.0 + 2.0 ** -8) == 1.0                      # tie -> even (down)
    assert brute.bf16_rne(1.0 + 3 * 2.0 ** -8) == 1.0 + 2 * 2.0 ** -7   # tie -> even (up)
    assert brute.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert brute.bf16_rne(-(2.0 - 2.0 ** -9)) == -2.0                  # carry into the exponent
    # a binary64 value just above a tie that fp32 would round to the tie first
    v = struct.unpack("<d", struct.pack("<Q", 0x3FF0100000000001))[0]   # 1 + 2**-8 + 2**-52
    assert brute.bf16_rne(v) == 1.0 + 2.0 ** -7
    # and the oracle's rounding agrees with this independent one on fp64 inputs
    y = np.random.default_rng(1).standard_normal(5000) * 10.0 ** np.random.default_rng(2).uniform(-8, 8, 5000)
    np.testing.assert_array_equal(D.bf16_round(y), [brute.bf16_rne(v) for v in y])


CASES = [(9, 0), (9, 6), (0, 0), (3, 3), (11, 2)]


@pytest.mark.parametrize("hc,ctx_norm", [(1, 0), (4, 1), (4, 0), (1, 1)])
def test_draft_block_matches_brute_force_exact_and_mirror(hc, ctx_norm):
    cfg = _small(hc_streams=hc, ctx_norm=ctx_norm)
    W = _f64_weights(cfg, seed=3 + hc + ctx_norm)
    taps = [t.numpy().astype(np.float64) for t in synth.make_taps(cfg, 12, seed=3, outliers=False)]
    tokens = [7, 63, 63]
    for mode in ("exact", "mirror"):
        for pos, vf in CASES:
            got = D.draft_block(cfg, W, taps, tokens, pos, vf, mode=mode)
            z, logits = brute.draft(cfg, W, taps, tokens, pos, vf, mirror=(mode == "mirror"))
            np.testing.assert_allclose(got["z"], np.array(z), rtol=1e-10, atol=1e-12, err_msg=f"{mode} z {pos} {vf}")
            np.testing.assert_allclose(got["logits"], np.array(logits), rtol=1e-10, atol=1e-12,
                                       err_msg=f"{mode} logits {pos} {vf}")


def test_every_cast_point_is_pinned():
    """The comparison above has teeth: the brute force with any one cast point
    left unrounded differs from the oracle's mirror mode by far more than the
    1e-10 bound, and mirror differs from exact. So a cast point dropped, added
    or moved in the oracle fails the comparison."""
    cfg = _small(hc_streams=2, ctx_norm=1)
    W = _f64_weights(cfg, seed=4)
    taps = [t.numpy().astype(np.float64) for t in synth.make_taps(cfg, 12, seed=3, outliers=False)]
    tokens = [7, 63, 63]
    ref = D.draft_block(cfg, W, taps, tokens, 9, 0, mode="mirror")
    ex = D.draft_block(cfg, W, taps, tokens, 9, 0, mode="exact")
    scale = float(np.max(np.abs(ref["logits"])))
    assert np.max(np.abs(ref["logits"] - ex["logits"])) > 1e-4 * scale
    for name in brute.CAST_POINTS:
        z, lg = brute.draft(cfg, W, taps, tokens, 9, 0, mirror=True, skip=(name,))
        dz = float(np.max(np.abs(np.array(z) - ref["z"])))
        dl = float(np.max(np.abs(np.array(lg) - ref["logits"])))
        assert max(dz, dl) > 1e-6 * max(scale, 1.0), name


def _target_small():
    cfg = _small()
    tcfg = cfg.replace(n_layers=2)
    W = _f64_weights(tcfg, seed=11, embed_scale=25.0)
    return tcfg, W


@pytest.mark.parametrize("mode", ["exact", "mirror"])
def test_tiny_target_rows_match_scalar_causal_decoder(mode):
    tcfg, W = _target_small()
    tokens = [5, 17, 3, 40, 12, 9, 33]
    tgt = T.TinyTarget(tcfg, W, n_layers=2, mode=mode)
    ids, taps, logits = tgt.feed(tokens, 0, want_logits=True)
    bl, bt = brute.target_rows(tcfg, W, 2, tokens, mirror=(mode == "mirror"))
    np.testing.assert_allclose(logits, np.array(bl), rtol=1e-10, atol=1e-12)
    for l in range(2):   # taps come back as float32 rows
        np.testing.assert_array_equal(taps[l], np.array(bt[l], dtype=np.float32))
    # argmax of the brute-force logits, lowest index on ties
    assert ids == [int(np.argmax(np.array(r))) for r in bl]
    # the batched prefix path leaves the cache a row-by-row feed leaves
    tgt.reset()
    tgt.prefill(tokens[:5])
    ids2, _, lg2 = tgt.feed(tokens[5:], 5, want_logits=True)
    np.testing.assert_allclose(lg2, np.array(bl[5:]), rtol=1e-9, atol=1e-11)


def test_tiny_target_detects_a_wrong_position():
    """A target whose rows sat at shifted positions would not match: the
    causal decoder's outputs depend on relative positions within the prefix
    only, but a per-row offset (row i at i + i) does change them."""
    tcfg, W = _target_small()
    tokens = [5, 17, 3, 40]
    bl, _ = brute.target_rows(tcfg, W, 2, tokens, mirror=False)
    op = brute._Ops
    orig = op.rot
    try:
        op.rot = lambda self, vec, p: orig(self, vec, 2 * p)
        bad, _ = brute.target_rows(tcfg, W, 2, tokens, mirror=False)
    finally:
        op.rot = orig
    assert np.max(np.abs(np.array(bad) - np.array(bl))) > 1e-6
