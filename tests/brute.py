"""Scalar brute-force statements of the drafter round and of the tiny causal
target, written with explicit Python loops over plain float lists.

They are the independent pins of the oracle (``oracle/dflash.py``,
``oracle/target.py``): nothing here calls the oracle or shares its helpers. The
bf16 rounding used at the cast points is its own integer implementation on the
IEEE-754 binary64 bit pattern (round to nearest, ties to even, at bit 45 of the
significand), not the oracle's frexp/rint route.

Sources for what is computed: "[RFC] DFlash", ExecuTorch PR #20840 ("DFlash
Overview", "Key Implementation Details", review threads on the Qwen3 modules the
drafter reuses, the bidirectional block and the rope offset); "feat: DFlash2
block-diffusion drafter for Qwen 3.8", Mference PR #22 ("What's here": sliding
context window, fp32 residual, shared LM head); "dflash: the chain verify builds
pipelined ...", mlx-serve PR #937 (hyper-connection stream mean).
"""
from __future__ import annotations

import math
import struct


def bf16_rne(x: float) -> float:
    """x rounded to bfloat16 (8 significant bits), ties to even, by integer
    arithmetic on the binary64 bits. Only normal bf16 results occur in the tests
    (an assertion guards the exponent range)."""
    x = float(x)
    if x == 0.0 or not math.isfinite(x):
        return x
    bits = struct.unpack("<Q", struct.pack("<d", x))[0]
    exp = (bits >> 52) & 0x7FF
    assert 1023 - 126 <= exp <= 1023 + 127, f"value {x!r} outside the normal bf16 range"
    drop = 52 - 7                        # significand bits below bf16's seven fraction bits
    low = bits & ((1 << drop) - 1)
    top = bits >> drop
    half = 1 << (drop - 1)
    if low > half or (low == half and (top & 1)):
        top += 1                         # a carry into the exponent is the correct result
    return struct.unpack("<d", struct.pack("<Q", top << drop))[0]


def _ident(x: float) -> float:
    return x


def _lists(W):
    out = {}
    for k, v in W.items():
        if isinstance(v, list):
            out[k] = [t.tolist() for t in v]
        else:
            out[k] = v.tolist()
    return out


class _Ops:
    def __init__(self, cfg, mirror: bool):
        self.cfg = cfg
        self.r = bf16_rne if mirror else _ident

    def norm(self, vec, g):
        ms = sum(x * x for x in vec) / len(vec)
        inv = 1.0 / math.sqrt(ms + self.cfg.rms_eps)
        return [g[i] * (vec[i] * inv) for i in range(len(vec))]

    @staticmethod
    def matvec(Wm, vec, r0, r1):
        return [sum(Wm[r][c] * vec[c] for c in range(len(vec))) for r in range(r0, r1)]

    def rot(self, vec, p):
        hd = len(vec)
        half = hd // 2
        out = list(vec)
        for k in range(half):
            ang = p * self.cfg.rope_theta ** (-2.0 * k / hd)
            z = complex(vec[k], vec[k + half]) * complex(math.cos(ang), math.sin(ang))
            out[k], out[k + half] = z.real, z.imag
        return out

    def attend(self, q, keys, vals):
        s = [sum(q[d] * kk[d] for d in range(len(q))) / math.sqrt(len(q)) for kk in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = sum(e)
        return [sum(e[t] * vals[t][d] for t in range(len(e))) / tot for d in range(len(q))]


CAST_POINTS = ("x", "c", "kv_ctx", "a", "qkv", "o", "a2", "act", "z")


def draft(cfg, W, taps, tokens, pos: int, valid_from: int, mirror: bool, skip=()):
    """One request's draft block, loops only. Returns (z [B][H], logits of
    rows 1..B-1 [B-1][V]). ``taps[t][p]`` is the fp32 tap row of absolute
    position p (hc_streams stream-major blocks of tap_hidden values).

    With ``mirror`` every value is rounded to bf16 at the cast points named in
    CAST_POINTS: the fc input x, the context hidden c, the context K/V, the
    input-normed rows a, the block's Q/K/V after head norm + RoPE, the
    attention output o, the post-attention-normed rows a2, SiLU(gate)*up and
    the final-normed rows z. ``skip`` leaves the named ones unrounded."""
    W = _lists(W)
    op = _Ops(cfg, mirror)
    rr = {name: (_ident if name in skip else op.r) for name in CAST_POINTS}
    H, nq, nkv, hd, F = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    Ht, hc = cfg.tap_hidden, cfg.hc_streams
    B = len(tokens)
    lo = max(valid_from, pos - cfg.window, 0)
    ctx = list(range(lo, pos))

    # context hidden: hc mean of each tap, concat in tap order, fc, optional norm
    cvec = []
    for p in ctx:
        x = []
        for t in range(cfg.n_taps):
            row = [float(v) for v in taps[t][p]]
            for col in range(Ht):
                x.append(rr["x"](sum(row[s * Ht + col] for s in range(hc)) / hc))
        c = op.matvec(W["fc"], x, 0, H)
        if cfg.ctx_norm:
            c = op.norm(c, W["ctx_norm"])
        cvec.append([rr["c"](v) for v in c])

    h = [list(W["embed"][t]) for t in tokens]
    grp = nq // nkv
    for l in range(cfg.n_layers):
        wqkv = W["wqkv"][l]
        koff, voff = nq * hd, (nq + nkv) * hd
        K = [[None] * (len(ctx) + B) for _ in range(nkv)]
        V = [[None] * (len(ctx) + B) for _ in range(nkv)]
        for n, p in enumerate(ctx):       # context rows: no input norm, k norm + rope at p
            for g in range(nkv):
                k = op.matvec(wqkv, cvec[n], koff + g * hd, koff + (g + 1) * hd)
                K[g][n] = [rr["kv_ctx"](v) for v in op.rot(op.norm(k, W["k_norm"][l]), p)]
                V[g][n] = [rr["kv_ctx"](v) for v in op.matvec(wqkv, cvec[n], voff + g * hd, voff + (g + 1) * hd)]
        a = [[rr["a"](v) for v in op.norm(h[i], W["ln_in"][l])] for i in range(B)]
        Q = [[None] * B for _ in range(nq)]
        for i in range(B):                # block rows at pos + i
            for j in range(nq):
                q = op.matvec(wqkv, a[i], j * hd, (j + 1) * hd)
                Q[j][i] = [rr["qkv"](v) for v in op.rot(op.norm(q, W["q_norm"][l]), pos + i)]
            for g in range(nkv):
                k = op.matvec(wqkv, a[i], koff + g * hd, koff + (g + 1) * hd)
                K[g][len(ctx) + i] = [rr["qkv"](v) for v in op.rot(op.norm(k, W["k_norm"][l]), pos + i)]
                V[g][len(ctx) + i] = [rr["qkv"](v) for v in op.matvec(wqkv, a[i], voff + g * hd, voff + (g + 1) * hd)]
        for i in range(B):                # every query sees every key: no mask
            o = []
            for j in range(nq):
                g = j // grp
                o.extend(rr["o"](v) for v in op.attend(Q[j][i], K[g], V[g]))
            y = op.matvec(W["wo"][l], o, 0, H)
            h[i] = [h[i][c] + y[c] for c in range(H)]
        for i in range(B):
            a2 = [rr["a2"](v) for v in op.norm(h[i], W["ln_post"][l])]
            gate = op.matvec(W["wgu"][l], a2, 0, F)
            up = op.matvec(W["wgu"][l], a2, F, 2 * F)
            act = [rr["act"](gate[f] / (1.0 + math.exp(-gate[f])) * up[f]) for f in range(F)]
            y = op.matvec(W["wd"][l], act, 0, H)
            h[i] = [h[i][c] + y[c] for c in range(H)]
    z = [[rr["z"](v) for v in op.norm(h[i], W["final_norm"])] for i in range(B)]
    logits = [op.matvec(W["lm_head"], z[i], 0, cfg.vocab) for i in range(1, B)]
    return z, logits


def target_rows(cfg, W, n_layers: int, tokens, mirror: bool):
    """A causal Qwen3-shaped decoder over ``tokens`` at positions 0, 1, ...,
    loops only: row i attends to rows 0..i. Returns (logits [n][V], taps
    [n_layers][n][H]) where taps are the residual rows after each layer."""
    W = _lists(W)
    op = _Ops(cfg, mirror)
    r = op.r
    H, nq, nkv, hd, F = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    grp = nq // nkv
    n = len(tokens)
    h = [list(W["embed"][t]) for t in tokens]
    taps = []
    for l in range(n_layers):
        wqkv = W["wqkv"][l]
        koff, voff = nq * hd, (nq + nkv) * hd
        a = [[r(v) for v in op.norm(h[i], W["ln_in"][l])] for i in range(n)]
        Q = [[[r(v) for v in op.rot(op.norm(op.matvec(wqkv, a[i], j * hd, (j + 1) * hd), W["q_norm"][l]), i)]
               for i in range(n)] for j in range(nq)]
        K = [[[r(v) for v in op.rot(op.norm(op.matvec(wqkv, a[i], koff + g * hd, koff + (g + 1) * hd),
                                             W["k_norm"][l]), i)]
              for i in range(n)] for g in range(nkv)]
        V = [[[r(v) for v in op.matvec(wqkv, a[i], voff + g * hd, voff + (g + 1) * hd)] for i in range(n)]
             for g in range(nkv)]
        for i in range(n):
            o = []
            for j in range(nq):
                g = j // grp
                o.extend(r(v) for v in op.attend(Q[j][i], K[g][:i + 1], V[g][:i + 1]))
            y = op.matvec(W["wo"][l], o, 0, H)
            h[i] = [h[i][c] + y[c] for c in range(H)]
            a2 = [r(v) for v in op.norm(h[i], W["ln_post"][l])]
            gate = op.matvec(W["wgu"][l], a2, 0, F)
            up = op.matvec(W["wgu"][l], a2, F, 2 * F)
            act = [r(gate[f] / (1.0 + math.exp(-gate[f])) * up[f]) for f in range(F)]
            y = op.matvec(W["wd"][l], act, 0, H)
            h[i] = [h[i][c] + y[c] for c in range(H)]
        taps.append([list(row) for row in h])
    logits = [op.matvec(W["lm_head"], [r(v) for v in op.norm(h[i], W["final_norm"])], 0, cfg.vocab)
              for i in range(n)]
    return logits, taps
