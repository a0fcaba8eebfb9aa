"""Pins of the oracle's elementwise numerics against library routines, closed
forms and brute force (no GPU)."""
import math

import numpy as np
import pytest
import torch

from oracle import dflash as D


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        rng.standard_normal(2000) * 1e-39,            # fp32 subnormal range
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38]),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = D.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_round_ties_to_even_bit_patterns():
    # 1 + 2**-8 is halfway between 1 and 1 + 2**-7: ties go to the even significand (1.0)
    assert D.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3 * 2**-8 is halfway between 1 + 2**-7 (odd) and 1 + 2**-6 (even)
    assert D.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above the tie rounds up
    assert D.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    # exactly representable values are fixed points
    for v in (0.5, 3.0, -7.5, 2.0 ** -126, 2.0 ** -133, 2.0 ** 127):
        assert D.bf16_round(v) == v
    # smallest subnormal: half of it rounds to zero (tie to even), 0.75 of it rounds up
    assert D.bf16_round(2.0 ** -134) == 0.0
    assert D.bf16_round(0.75 * 2.0 ** -133) == 2.0 ** -133
    # overflow past the largest finite bf16 ((2 - 2**-7) * 2**127)
    assert D.bf16_round(2.0 ** 128 * (1 - 2.0 ** -10)) == math.inf
    assert np.isnan(D.bf16_round(np.nan))
    assert D.bf16_round(-np.inf) == -np.inf


def test_bf16_round_random_ties_against_torch():
    # construct exact midpoints between neighbouring bf16 values (representable in fp32)
    rng = np.random.default_rng(1)
    bits = rng.integers(0x0080, 0x7F00, 5000).astype(np.uint32) << 16
    lo = bits.view(np.float32).astype(np.float64)
    mid = (lo + (bits + 0x10000).view(np.float32).astype(np.float64)) / 2
    ref = torch.from_numpy(mid.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(D.bf16_round(mid), ref.astype(np.float64))


# ------------------------------------------------------------------ RMSNorm, SiLU

def test_rmsnorm_closed_forms():
    eps = 1e-6
    for c in (0.3, -2.0, 17.0):
        x = np.full((3, 64), c)
        g = np.linspace(0.5, 1.5, 64)
        np.testing.assert_allclose(D.rmsnorm(x, g, eps), np.broadcast_to(g * c / math.sqrt(c * c + eps), x.shape), rtol=1e-15)
    # one nonzero entry a among n: output a / sqrt(a^2/n + eps) there, 0 elsewhere
    x = np.zeros(16)
    x[5] = 3.0
    out = D.rmsnorm(x, np.ones(16), 0.0)
    assert out[5] == pytest.approx(4.0, rel=1e-15)      # 3 / sqrt(9/16)
    assert np.count_nonzero(out) == 1
    # with eps = 0, scale invariant
    r = np.random.default_rng(0).standard_normal((4, 32))
    np.testing.assert_allclose(D.rmsnorm(5.0 * r, np.ones(32), 0.0), D.rmsnorm(r, np.ones(32), 0.0),
                               rtol=1e-14)


def test_silu_closed_forms():
    assert D.silu(0.0) == 0.0
    assert D.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert D.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert abs(D.silu(-50.0)) < 1e-19
    x = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(D.silu(x) - D.silu(-x), x, atol=1e-14)   # x*s(x) - (-x)*s(-x) = x
    np.testing.assert_allclose(D.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ RoPE

def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(2)
    hd, theta = 64, 1e6
    x = rng.standard_normal((3, 5, hd))
    pos = np.array([0, 1, 7, 1000, 16383])
    got = D.rope(x, pos, theta)
    half = hd // 2
    z = x[..., :half] + 1j * x[..., half:]
    freqs = theta ** (-np.arange(0, hd, 2) / hd)
    rot = z * np.exp(1j * pos[:, None] * freqs[None, :])
    np.testing.assert_allclose(got[..., :half], rot.real, atol=1e-12)
    np.testing.assert_allclose(got[..., half:], rot.imag, atol=1e-12)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(3)
    hd = 128
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    np.testing.assert_array_equal(D.rope(q, [0], 1e6), q)
    for p in (5, 4096, 16400):
        np.testing.assert_allclose(np.linalg.norm(D.rope(q, [p], 1e6)), np.linalg.norm(q), rtol=1e-13)
    # <R(p1) q, R(p2) k> depends only on p1 - p2
    d1 = float(np.sum(D.rope(q, [100], 1e6) * D.rope(k, [37], 1e6)))
    d2 = float(np.sum(D.rope(q, [4163], 1e6) * D.rope(k, [4100], 1e6)))
    assert d1 == pytest.approx(d2, rel=1e-9, abs=1e-9)


# ------------------------------------------------------------------ hc stream mean

def test_hc_mean_explicit_loop_identity_and_identical_streams():
    rng = np.random.default_rng(4)
    n, hc, w = 3, 4, 10
    t = rng.standard_normal((n, hc * w))
    ref = np.zeros((n, w))
    for r in range(n):
        for k in range(w):
            ref[r, k] = sum(t[r, s * w + k] for s in range(hc)) / hc
    np.testing.assert_allclose(D.hc_mean(t, hc, w), ref, rtol=1e-15)
    np.testing.assert_array_equal(D.hc_mean(t[:, :w], 1, w), t[:, :w])
    one = rng.standard_normal((n, w))
    np.testing.assert_allclose(D.hc_mean(np.tile(one, (1, hc)), hc, w), one, rtol=1e-15)


# ------------------------------------------------------------------ attention

def _brute_attention(q, k, v):
    """Scalar loops: scores, max-subtracted exponentials, weighted sum."""
    nq, nb, hd = q.shape
    nkv, nk, _ = k.shape
    grp = nq // nkv
    out = np.zeros((nb, nq, hd))
    for j in range(nq):
        g = j // grp
        for i in range(nb):
            s = [sum(q[j, i, d] * k[g, t, d] for d in range(hd)) / math.sqrt(hd) for t in range(nk)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = sum(e)
            for d in range(hd):
                out[i, j, d] = sum(e[t] * v[g, t, d] for t in range(nk)) / tot
    return out


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 3, 8))
    k = rng.standard_normal((2, 7, 8))
    v = rng.standard_normal((2, 7, 8))
    np.testing.assert_allclose(D.attention(q, k, v), _brute_attention(q, k, v), rtol=1e-12, atol=1e-12)


def test_attention_matches_sdpa_fp64_gqa():
    rng = np.random.default_rng(6)
    nq, nkv, nb, nk, hd = 8, 2, 5, 19, 16
    q = rng.standard_normal((nq, nb, hd))
    k = rng.standard_normal((nkv, nk, hd))
    v = rng.standard_normal((nkv, nk, hd))
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(nq // nkv, 0)
    tv = torch.from_numpy(v).repeat_interleave(nq // nkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=False)
    np.testing.assert_allclose(D.attention(q, k, v), ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_attention_gqa_equals_mha_with_duplicated_heads():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((6, 4, 8))
    k = rng.standard_normal((3, 9, 8))
    v = rng.standard_normal((3, 9, 8))
    mha = D.attention(q, np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0))
    np.testing.assert_array_equal(D.attention(q, k, v), mha)


# ------------------------------------------------------------------ top-k

def test_topk_against_sorted_with_ties():
    rng = np.random.default_rng(8)
    x = rng.integers(0, 5, (20, 40)).astype(np.float64)      # many ties
    for k in (1, 3, 16):
        ids, vals = D.topk(x, k)
        for r in range(x.shape[0]):
            ref = sorted(range(x.shape[1]), key=lambda i: (-x[r, i], i))[:k]
            assert list(ids[r]) == ref
            np.testing.assert_array_equal(vals[r], x[r, ref])
    assert D.topk(np.array([[1.0, 3.0, 3.0, 2.0]]), 1)[0][0, 0] == 1


# ------------------------------------------------------------------ accept-profile identity

def test_tokens_per_round_reproduces_printed_figures():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "accept_profile.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        tpr = D.tokens_per_round(np.array(case["profile_pct"]) / 100.0)
        assert tpr == pytest.approx(case["tokens_per_round"], abs=0.005), case["name"]
