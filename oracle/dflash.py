"""fp64 oracle of the DFlash drafter round (test infrastructure only).

Sources (the three pages this build follows):
  [P1] "feat: DFlash2 block-diffusion drafter for Qwen 3.8 (opt-in, byte-identical)",
       Mference PR #22 - commit messages and the PR body ("What's here", "Gates",
       "Measured").
  [P2] "dflash: the chain verify builds pipelined and defers the qwen4 PLE gather,
       as the MTP verify does", mlx-serve PR #937 - the hyper-connection-stream
       commit.
  [P3] "[RFC] DFlash", ExecuTorch PR #20840 - "DFlash Overview", "Key
       Implementation Details", the review threads and the author's reply.

What the round computes, step by step, and the readings taken where the pages
leave a step open, are in each function's docstring. Everything is fp64. In
``mirror`` mode values are rounded to bf16 at the cast points of the GPU numerics
contract (listed in ``CAST_POINTS``); in ``exact`` mode no rounding happens.

This module shares no code with the HIP path and imports nothing from it.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

CAST_POINTS = (
    "fc input x (hc-mean of the taps, concatenated)",
    "ctx hidden c after fc (and the optional ctx RMSNorm)",
    "every RMSNorm output that feeds a matrix product",
    "Q and K after head norm + RoPE, V after its projection (ctx ring included)",
    "attention output O before the o projection",
    "SiLU(gate) * up before the down projection",
    "final normed hidden z before the LM head",
)


# ----------------------------------------------------------------------------- numerics

def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps the fp32 exponent range and 8 significant bits. For |x| in
    [2**E, 2**(E+1)) the spacing of representable values is 2**(E-7); below the
    smallest normal (2**-126) the spacing stays 2**-133 (subnormals). Rounding is
    ``rint(x / spacing) * spacing``; ``np.rint`` rounds halves to even. Results
    at or beyond 2**128 overflow to +-inf. Pinned by tests against torch's
    fp32->bf16 conversion and against hand-computed bit patterns.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0)
    if not np.any(finite):
        return out
    xf = x[finite]
    _, e = np.frexp(xf)                 # xf = m * 2**e, 0.5 <= |m| < 1  ->  E = e - 1
    E = np.maximum(e - 1, -126)
    spacing = np.ldexp(1.0, E - 7)
    r = np.rint(xf / spacing) * spacing
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def _rnd(mode: str):
    if mode == "mirror":
        return bf16_round
    if mode == "exact":
        return lambda v: np.asarray(v, dtype=np.float64)
    raise ValueError(f"unknown mode {mode!r}")


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rmsnorm(x, g, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: g * x / sqrt(mean(x**2) + eps).

    The drafter layers reuse the Qwen3 RMSNorm ([P3] review thread on reusing the
    Hugging Face modules; the author's swap to ``F.rms_norm`` keeps its order of
    operations). Pinned by closed forms (constant rows, scaling invariance).
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return _f64(g) * (x / np.sqrt(ms + eps))


def silu(x) -> np.ndarray:
    """x * sigmoid(x), the SwiGLU gate nonlinearity of the Qwen3 MLP [P3]."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """theta ** (-2k / head_dim) for k = 0 .. head_dim/2 - 1."""
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * k / head_dim)


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of the last axis (the Qwen3 rotary embedding
    the drafter reuses, [P3]).

    x: [..., n, hd] with positions [n]. For k < hd/2 the pair (x[k], x[k+hd/2])
    is rotated by the angle position * theta**(-2k/hd). Block rows sit at
    pos + i, so the offset moves with the context length ([P3] review thread on
    the rope op: the offset has to shift with context length). Pinned by the
    complex-multiplication form, norm preservation and the relative-position
    identity.
    """
    x = _f64(x)
    hd = x.shape[-1]
    half = hd // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inv_freq(hd, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def hc_mean(tap_rows, hc: int, width: int) -> np.ndarray:
    """Per-token mean of ``hc`` hyper-connection streams laid out stream-major on
    the last axis ([n, hc*width] -> [n, width]): reshape then mean over the
    stream axis, as the hc commit of [P2] describes. hc = 1 is the identity.
    Pinned by an explicit loop, hc = 1 and identical-stream tests.
    """
    t = _f64(tap_rows)
    return t.reshape(t.shape[0], hc, width).mean(axis=1)


def softmax(s, axis=-1) -> np.ndarray:
    s = _f64(s)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q, k, v) -> np.ndarray:
    """Grouped-query attention with no mask.

    q: [nq, nb, hd] (block queries), k, v: [nkv, nk, hd] (keys = [ctx | block]).
    Query head j reads kv head j // (nq // nkv) (contiguous head groups, as in
    Qwen3 GQA). Scores are scaled by 1/sqrt(hd); softmax runs over every key: the
    block is bidirectional ([P1] "What's here"; [P3] review: the causal proposal
    mask was a bug for this checkpoint). Returns [nb, nq, hd].
    Pinned by brute-force loops, SDPA in fp64 and MHA equivalence.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, nb, hd = q.shape
    nkv = k.shape[0]
    grp = nq // nkv
    out = np.empty((nb, nq, hd))
    for j in range(nq):
        g = j // grp
        s = q[j] @ k[g].T / math.sqrt(hd)
        out[:, j, :] = softmax(s, axis=-1) @ v[g]
    return out


# ----------------------------------------------------------------------------- drafter

def window_bounds(pos: int, valid_from: int, window: int):
    """Committed context rows the block attends to: [max(valid_from, pos - W, 0), pos).

    Reading: the window counts context rows only and one key set is shared by all
    block queries ([P1] "What's here": attention over a sliding context window
    followed by the bidirectional block). Only valid rows are read, as in the
    cached drafter the [P3] author shipped (narrowing to valid rows instead of a
    masked full buffer).
    """
    lo = max(int(valid_from), int(pos) - int(window), 0)
    return lo, int(pos)


def ctx_hidden(cfg, W, taps: Sequence, lo: int, hi: int, mode: str = "mirror") -> np.ndarray:
    """Context hidden rows for positions [lo, hi): [hi-lo, H].

    Step 1 of the round ([P3] "Key Implementation Details", Phase 1: the target
    returns its selected layers' hidden rows concatenated; the drafter's fc maps
    them to its hidden size): x_p = concat_t hc_mean(tap_t[p]), cast to bf16;
    c_p = W_fc x_p; with ``ctx_norm`` an RMSNorm with gain ``ctx_norm`` follows
    (reading: off by default, the pages name only the projection); c is cast to
    bf16. ``taps[t]`` is indexed by absolute position. Pinned by the scalar
    brute force (hc 1 and 4, ctx norm on and off), by linearity and by one-hot
    tap columns.
    """
    rnd = _rnd(mode)
    parts = [hc_mean(np.asarray(taps[t])[lo:hi], cfg.hc_streams, cfg.tap_hidden)
             for t in range(cfg.n_taps)]
    x = rnd(np.concatenate(parts, axis=1)) if parts else np.zeros((0, cfg.tap_width))
    c = x @ _f64(W["fc"]).T
    if cfg.ctx_norm:
        c = rmsnorm(c, W["ctx_norm"], cfg.rms_eps)
    return rnd(c)


def _split_qkv(cfg, w):
    w = _f64(w)
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    return w[: nq * hd], w[nq * hd: (nq + nkv) * hd], w[(nq + nkv) * hd:]


def kv_project(cfg, W, layer: int, c, positions, mode: str = "mirror"):
    """Layer ``layer``'s K/V of context rows: K = RoPE(knorm(W_k c), p), V = W_v c.

    Reading of the garbled [P3] "DFlash Overview" sentence on conditioning: the
    tap-derived context enters every draft layer as extra key/value rows
    projected by that layer's own W_k and W_v ([P1] "KV-injected target taps";
    attention over [context | block]). Context rows skip the layer's input
    RMSNorm. Returns K, V as [nkv, n, hd], bf16-cast in mirror mode.
    """
    rnd = _rnd(mode)
    nkv, hd = cfg.n_kv_heads, cfg.head_dim
    _, wk, wv = _split_qkv(cfg, W["wqkv"][layer])
    c = _f64(c)
    n = c.shape[0]
    k = (c @ wk.T).reshape(n, nkv, hd)
    v = (c @ wv.T).reshape(n, nkv, hd)
    k = rmsnorm(k, W["k_norm"][layer], cfg.rms_eps)
    k = rope(k.transpose(1, 0, 2), positions, cfg.rope_theta)
    return rnd(k), rnd(v.transpose(1, 0, 2))


def draft_block(cfg, W, taps: Sequence, tokens, pos: int, valid_from: int = 0,
                mode: str = "mirror", want_intermediates: bool = False) -> Dict[str, object]:
    """One request's masked-block draft forward (uncached definition).

    The block (token 0 known, the rest ``mask_id``) runs through every draft
    layer in one forward ([P3] "DFlash Overview"; [P1] "What's here"). The
    context K/V is recomputed from the committed taps in the window each call,
    the uncached drafter of [P3]'s first version; the GPU's incremental ring must
    agree with it (the [P3] reviewer asked for cached-vs-uncached parity).

    Per layer (Qwen3 decoder layer, reused by [P3]'s drafter):
      a = RMSNorm(h; ln_in) -> Q, K_b, V_b -> q/k head RMSNorm -> RoPE(pos + i)
      keys = [K_ctx ; K_b], values = [V_ctx ; V_b], no mask, GQA
      h += W_o O ; a2 = RMSNorm(h; ln_post) ; h += W_d(SiLU(W_g a2) * W_u a2)
    The residual h stays fp64 here (fp32 on the GPU: [P1] "What's here" keeps an
    fp32 residual because o/down outputs overflow fp16 on outlier channels).
    Head: z = RMSNorm(h; final_norm); logits_i = W_lm z_i for rows 1..B-1 (each
    mask row predicts the token at its own position; row 0 is the known token).

    Returns a dict with ``logits`` [B-1, V], ``z`` [B, H] and, when
    ``want_intermediates``, ``h`` [B, H] and per-layer ``ctx_k``/``ctx_v``.

    Pinned by a scalar brute force written with loops and its own bf16 rounding
    (exact and mirror modes, 1 or 4 hc streams, ctx norm on and off; every cast
    point checked to matter), and by the invariants the pages fix
    (bidirectional block, sliding window, rope offset, GQA = MHA, context
    length 0 = textbook attention).
    """
    rnd = _rnd(mode)
    tokens = np.asarray(tokens, dtype=np.int64)
    B = tokens.shape[0]
    H, nq, nkv, hd = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    lo, hi = window_bounds(pos, valid_from, cfg.window)
    c = ctx_hidden(cfg, W, taps, lo, hi, mode)
    ctx_pos = np.arange(lo, hi)
    blk_pos = pos + np.arange(B)

    h = _f64(W["embed"])[tokens]                 # embed scale 1 (Qwen)
    inter = {"ctx_k": [], "ctx_v": [], "ctx_c": c, "lo": lo, "hi": hi}
    for l in range(cfg.n_layers):
        a = rnd(rmsnorm(h, W["ln_in"][l], cfg.rms_eps))
        wq, wk, wv = _split_qkv(cfg, W["wqkv"][l])
        q = (a @ wq.T).reshape(B, nq, hd)
        kb = (a @ wk.T).reshape(B, nkv, hd)
        vb = (a @ wv.T).reshape(B, nkv, hd)
        q = rmsnorm(q, W["q_norm"][l], cfg.rms_eps)
        kb = rmsnorm(kb, W["k_norm"][l], cfg.rms_eps)
        q = rnd(rope(q.transpose(1, 0, 2), blk_pos, cfg.rope_theta))      # [nq, B, hd]
        kb = rnd(rope(kb.transpose(1, 0, 2), blk_pos, cfg.rope_theta))    # [nkv, B, hd]
        vb = rnd(vb.transpose(1, 0, 2))
        kc, vc = kv_project(cfg, W, l, c, ctx_pos, mode)
        inter["ctx_k"].append(kc)
        inter["ctx_v"].append(vc)
        keys = np.concatenate([kc, kb], axis=1)
        vals = np.concatenate([vc, vb], axis=1)
        o = rnd(attention(q, keys, vals).reshape(B, nq * hd))
        h = h + o @ _f64(W["wo"][l]).T
        a2 = rnd(rmsnorm(h, W["ln_post"][l], cfg.rms_eps))
        wgu = _f64(W["wgu"][l])
        g = a2 @ wgu[: cfg.ffn].T
        u = a2 @ wgu[cfg.ffn:].T
        act = rnd(silu(g) * u)
        h = h + act @ _f64(W["wd"][l]).T
    z = rnd(rmsnorm(h, W["final_norm"], cfg.rms_eps))
    logits = z[1:] @ _f64(W["lm_head"]).T
    out = {"logits": logits, "z": z}
    if want_intermediates:
        inter["h"] = h
        out.update(inter)
    return out


# ----------------------------------------------------------------------------- selection

def topk(logits, k: int):
    """Top-k per row ordered by (value descending, index ascending).

    k = 1 is argmax with the lowest index on ties. [P1] keeps top-16 candidate
    lists per block position; [P3]'s driver takes the argmax. Returns
    (ids [n, k] int64, values [n, k]). Pinned against a stable argsort.
    """
    x2 = np.atleast_2d(_f64(logits))
    n, V = x2.shape
    ids = np.empty((n, k), dtype=np.int64)
    for r in range(n):
        # lexsort orders by the last key first: -value ascending, then index ascending
        ids[r] = np.lexsort((np.arange(V), -x2[r]))[:k]
    vals = np.take_along_axis(x2, ids, axis=1)
    return ids, vals


def accept(draft, verify, eos_id: int = -1, budget: Optional[int] = None) -> Dict[str, object]:
    """First-mismatch acceptance with the bonus token ([P3] "Phase 3" and the
    review note on the first-mismatch helper: draft ids have length B-1, verify
    ids length B, so the verify id at the accept index always exists).

      acc     = first j with draft[j] != verify[j], else B-1
      emitted = draft[:acc] + [verify[acc]]
      EOS     : keep up to and including its first occurrence (reviewer note on
                the driver's EOS truncation), if eos_id >= 0
      budget  : keep at most max(budget, 1) tokens (the remaining generation
                budget; reading: a verified round always emits the target token)
      acc     = min(acc, n_emit - 1) (the accepted count after truncation)
    The committed context rows are the first n_emit verify rows ([P3]: only
    ``new_hidden[:, :len(new_tokens)]`` extends the context). Pinned by an
    exhaustive characterization test.
    """
    d = [int(t) for t in draft]
    v = [int(t) for t in verify]
    assert len(v) == len(d) + 1
    acc = len(d)
    for j in range(len(d)):
        if d[j] != v[j]:
            acc = j
            break
    emitted = d[:acc] + [v[acc]]
    if eos_id >= 0 and eos_id in emitted:
        emitted = emitted[: emitted.index(eos_id) + 1]
    if budget is not None:
        emitted = emitted[: max(int(budget), 1)]
    n = len(emitted)
    return {"acc": min(acc, n - 1), "emitted": emitted, "n_emit": n}


def next_block(emitted: List[int], block: int, mask_id: int) -> List[int]:
    """The next round's block: the last emitted token, then mask ids."""
    return [int(emitted[-1])] + [int(mask_id)] * (block - 1)


def block_len(block_size: int, max_new: int, n_generated: int, max_seq: int, position: int) -> int:
    """Block length of the next round: the configured block, shrunk so that a
    round can neither emit past the generation budget nor run past the sequence
    capacity ("[RFC] DFlash": the review item asking for a dynamic block length
    and the author's reply, which bounds it by 1 <= block_len <= block size).

      block_len = min(block_size, max_new - n_generated, max_seq - position)

    A value below 1 means no round is left; 1 is a target-only step (no draft
    rows: the accept emits the target's token).
    """
    return min(int(block_size), int(max_new) - int(n_generated), int(max_seq) - int(position))


def tokens_per_round(profile: Sequence[float]) -> float:
    """Mean tokens per round from a per-draft-position accept profile.

    A round emits acc + 1 tokens, and E[acc] = sum_i P(acc >= i); the profile's
    entry i is P(acc >= i+1). ([P1] "Measured" prints both the profile and the
    tokens per round, which this identity links.)
    """
    return 1.0 + float(np.sum(np.asarray(profile, dtype=np.float64)))


# ----------------------------------------------------------------------------- INT4

def int4_unpack(packed, scales, K: int) -> np.ndarray:
    """Exact fp64 values q*s of a packed INT4 g64 matrix.

    Layout (the library's documented format): per row, K/2 bytes read as
    little-endian 32-bit words; in the 128-wide chunk c, word 4*j + s holds the
    values k = 128c + 32s + 8j + e (e = 0..7) as u = q + 8, value e in nibble e/2
    (even e) or 4 + (e-1)/2 (odd e). Scales are fp16 [N, K/64]. The weight format
    is the INT4-projection workload's (symmetric, groups of 64, fp16 scales); [P1]
    quantizes its drafter's projections to INT4 at load ("What's here").
    """
    b = np.asarray(packed, dtype=np.uint8)
    N = b.shape[0]
    words = b.reshape(N, K // 8, 4).astype(np.uint32)
    words = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    q = np.empty((N, K), dtype=np.float64)
    for c in range(K // 128):
        for j in range(4):
            for s in range(4):
                w = words[:, c * 16 + 4 * j + s]
                for e in range(8):
                    nib = e // 2 if e % 2 == 0 else 4 + (e - 1) // 2
                    u = (w >> np.uint32(4 * nib)) & np.uint32(0xF)
                    q[:, 128 * c + 32 * s + 8 * j + e] = u.astype(np.float64) - 8.0
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    return q * np.repeat(sc, 64, axis=1)


def dequantize(W) -> Dict[str, object]:
    """The weights an INT4-projection drafter computes with.

    Every projection that comes with ``<name>_scales`` (fc, wqkv, wo, wgu, wd)
    is replaced by its exact values q*s from ``int4_unpack``; embed, LM head and
    norm gains pass through unchanged (the INT4 workload keeps the LM head in
    bf16; [P1] quantizes the drafter's projections at load, "What's here"). The
    round itself is then the same definition as for bf16 weights.
    """
    out = dict(W)
    for name in ("fc", "wqkv", "wo", "wgu", "wd"):
        key = name + "_scales"
        if out.get(key) is None:
            continue
        if isinstance(W[name], list):
            out[name] = [int4_unpack(p, s, 2 * np.asarray(p).shape[1]) for p, s in zip(W[name], W[key])]
        else:
            out[name] = int4_unpack(W[name], W[key], 2 * np.asarray(W[name]).shape[1])
        del out[key]
    return out
