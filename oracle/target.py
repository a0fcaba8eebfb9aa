"""Tiny synthetic causal target and the speculative decoding loop (test infrastructure only).

The losslessness property ([P3] "[RFC] DFlash", ExecuTorch PR #20840, "Summary"
and "Test Plan": speculative output is token-for-token identical to greedy
decoding; [P1] "feat: DFlash2 block-diffusion drafter for Qwen 3.8", Mference
PR #22: every emitted byte is unchanged for any draft quality) is checked against
this target. It is a 2-layer Qwen3-shaped causal decoder in fp64 that shares the
drafter's embedding and LM head; its taps are the residual rows after each of
its layers (reading: the pages tap "selected target layers' hidden states"
without fixing which point inside the layer; the post-layer residual is the
plainest choice).

Batch invariance: every row - whether it comes from a single greedy step or
from a B-row verify pass - is computed by the same per-row routine against the
same cache contents, so the verify argmaxes equal the greedy ones bit for bit.
[P3]'s author traced an argmax flip to a kernel whose accumulation order changed
with batch size; computing rows one at a time rules that out here.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

from . import dflash as D


class TinyTarget:
    """fp64 causal decoder. ``weights`` holds per-layer lists like the drafter
    (wqkv, wo, wgu, wd, ln_in, ln_post, q_norm, k_norm), plus embed, lm_head and
    final_norm. ``cfg`` supplies the widths (the drafter's config)."""

    def __init__(self, cfg, weights: Dict[str, object], n_layers: int = 2, mode: str = "exact"):
        """``mode``: "exact" (fp64 throughout) or "mirror" (values rounded to bf16
        at the drafter's cast points: normed rows feeding products, Q/K after
        head norm + RoPE, V and the cached K/V, attention output, SiLU.up, the
        final normed row)."""
        self.cfg = cfg
        self.n_layers = n_layers
        self.rnd = D._rnd(mode)
        f = D._f64
        self.W = {
            "embed": f(weights["embed"]), "lm_head": f(weights["lm_head"]),
            "final_norm": f(weights["final_norm"]),
        }
        for name in ("wqkv", "wo", "wgu", "wd", "ln_in", "ln_post", "q_norm", "k_norm"):
            self.W[name] = [f(t) for t in weights[name][:n_layers]]
        self.reset()

    def reset(self):
        nkv, hd = self.cfg.n_kv_heads, self.cfg.head_dim
        self.k = [np.zeros((0, nkv, hd)) for _ in range(self.n_layers)]
        self.v = [np.zeros((0, nkv, hd)) for _ in range(self.n_layers)]

    @property
    def length(self) -> int:
        return self.k[0].shape[0]

    def _row(self, token: int, position: int):
        """One causal step: appends this row's K/V, returns (logits [V], taps [L][H]).
        Pinned, in exact and mirror modes, by a scalar causal decoder written with
        loops (row i attends to rows 0..i at positions 0..i)."""
        cfg, W = self.cfg, self.W
        nq, nkv, hd, eps = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
        assert position == self.length
        rnd = self.rnd
        h = W["embed"][int(token)].copy()
        taps = []
        for l in range(self.n_layers):
            a = rnd(D.rmsnorm(h, W["ln_in"][l], eps))
            wq, wk, wv = D._split_qkv(cfg, W["wqkv"][l])
            q = D.rmsnorm((wq @ a).reshape(nq, hd), W["q_norm"][l], eps)
            k = D.rmsnorm((wk @ a).reshape(nkv, hd), W["k_norm"][l], eps)
            v = rnd((wv @ a).reshape(nkv, hd))
            pos = np.array([position])
            q = rnd(D.rope(q[:, None, :], pos, cfg.rope_theta))       # [nq, 1, hd]
            k = rnd(D.rope(k[:, None, :], pos, cfg.rope_theta)[:, 0])
            self.k[l] = np.concatenate([self.k[l], k[None]], 0)
            self.v[l] = np.concatenate([self.v[l], v[None]], 0)
            o = rnd(D.attention(q, self.k[l].transpose(1, 0, 2), self.v[l].transpose(1, 0, 2)))
            h = h + W["wo"][l] @ o.reshape(nq * hd)
            a2 = rnd(D.rmsnorm(h, W["ln_post"][l], eps))
            g = W["wgu"][l][: cfg.ffn] @ a2
            u = W["wgu"][l][cfg.ffn:] @ a2
            h = h + W["wd"][l] @ rnd(D.silu(g) * u)
            taps.append(h.copy())
        logits = W["lm_head"] @ rnd(D.rmsnorm(h, W["final_norm"], eps))
        return logits, taps

    def feed(self, tokens: Sequence[int], start: int, want_logits: bool = False):
        """Rows for tokens at positions start.. (causal, one at a time).
        Returns (argmax ids [n], taps [n_layers][n, H] as float32), plus the
        fp64 logits [n, V] when ``want_logits``."""
        ids, taps, lg = [], [[] for _ in range(self.n_layers)], []
        for i, t in enumerate(tokens):
            logits, tr = self._row(t, start + i)
            ids.append(int(D.topk(logits, 1)[0][0, 0]))
            lg.append(logits)
            for l in range(self.n_layers):
                taps[l].append(tr[l])
        out = (ids, [np.asarray(t, dtype=np.float32).reshape(len(tokens), -1) for t in taps])
        return out + (np.asarray(lg),) if want_logits else out

    def prefill(self, tokens: Sequence[int]):
        """Append the cache rows of a prompt without logits or taps. The same
        per-row arithmetic as ``_row`` (cast points included), with the rows'
        projections done as one matrix product per weight and the causal
        attention of row i over cache rows [0, start + i]. Equal to feeding the
        tokens one at a time up to fp64 summation order; pinned against ``feed``."""
        cfg, W = self.cfg, self.W
        nq, nkv, hd, eps, F = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.ffn
        rnd = self.rnd
        start, n = self.length, len(tokens)
        pos = np.arange(start, start + n)
        h = W["embed"][np.asarray(tokens, dtype=np.int64)].copy()            # [n, H]
        for l in range(self.n_layers):
            a = rnd(D.rmsnorm(h, W["ln_in"][l], eps))
            wq, wk, wv = D._split_qkv(cfg, W["wqkv"][l])
            q = D.rmsnorm((a @ wq.T).reshape(n, nq, hd), W["q_norm"][l], eps)
            k = D.rmsnorm((a @ wk.T).reshape(n, nkv, hd), W["k_norm"][l], eps)
            v = rnd((a @ wv.T).reshape(n, nkv, hd))
            q = rnd(D.rope(q.transpose(1, 0, 2), pos, cfg.rope_theta))        # [nq, n, hd]
            k = rnd(D.rope(k.transpose(1, 0, 2), pos, cfg.rope_theta))        # [nkv, n, hd]
            self.k[l] = np.concatenate([self.k[l], k.transpose(1, 0, 2)], 0)
            self.v[l] = np.concatenate([self.v[l], v], 0)
            kc, vc = self.k[l].transpose(1, 0, 2), self.v[l].transpose(1, 0, 2)
            o = np.empty((n, nq, hd))
            for i in range(n):
                hi = start + i + 1
                o[i] = D.attention(q[:, i:i + 1, :], kc[:, :hi], vc[:, :hi])[0]
            h = h + rnd(o).reshape(n, nq * hd) @ W["wo"][l].T
            a2 = rnd(D.rmsnorm(h, W["ln_post"][l], eps))
            g = a2 @ W["wgu"][l][:F].T
            u = a2 @ W["wgu"][l][F:].T
            h = h + rnd(D.silu(g) * u) @ W["wd"][l].T

    def truncate(self, n: int):
        """Keep the first n cached rows (rollback after a verify pass)."""
        self.k = [k[:n] for k in self.k]
        self.v = [v[:n] for v in self.v]


def greedy(target: TinyTarget, prompt: Sequence[int], n_new: int, eos_id: int = -1) -> List[int]:
    """Plain greedy decoding: n_new tokens after the prompt (stops after EOS)."""
    target.reset()
    ids, _ = target.feed(prompt, 0)
    out = [ids[-1]]
    while len(out) < n_new and out[-1] != eos_id:
        nxt, _ = target.feed([out[-1]], target.length)
        out.append(nxt[0])
    return out


DraftFn = Callable[[List[int], int, int, List[np.ndarray]], Sequence[int]]


def speculative(target: TinyTarget, draft_fn: DraftFn, prompt: Sequence[int], n_new: int,
                block: int, window: int, mask_id: int, eos_id: int = -1, dynamic: bool = False,
                max_seq: Optional[int] = None) -> Dict[str, object]:
    """DFlash draft/verify loop ([P3] "Phase 3": draft a block, verify it with the
    target, accept to the first mismatch plus the target's token, roll the cache
    back; [P1]: verify stages the tap rows the drafter reads next).

    ``draft_fn(block_tokens, pos, valid_from, taps_by_position)`` returns B-1
    draft ids; taps_by_position[t] holds the committed tap rows [0, pos) of tapped
    layer t. With ``dynamic`` each round's block length is ``D.block_len`` of the
    remaining budget and of the sequence capacity ``max_seq`` (positions fed to
    the target stay below it); a length of 1 is a target-only step. Returns the
    emitted tokens, per-round accept lengths and block lengths.
    """
    target.reset()
    ids, taps = target.feed(prompt, 0)
    committed = [t.copy() for t in taps]
    pos = len(prompt)
    out = [ids[-1]]
    accepts, blocks = [], []
    cap = max_seq if max_seq is not None else pos + n_new + block
    while len(out) < n_new and out[-1] != eos_id:
        b = D.block_len(block, n_new, len(out), cap, pos) if dynamic else block
        if b < 1:
            break
        blk = D.next_block(out, b, mask_id)
        draft = [int(t) for t in draft_fn(blk, pos, 0, committed)] if b > 1 else []
        assert len(draft) == b - 1
        verify, vtaps = target.feed([blk[0]] + draft, pos)
        res = D.accept(draft, verify, eos_id=eos_id, budget=n_new - len(out))
        n = res["n_emit"]
        target.truncate(pos + n)
        committed = [np.concatenate([c, vt[:n]], 0) for c, vt in zip(committed, vtaps)]
        pos += n
        out.extend(res["emitted"])
        accepts.append(res["acc"])
        blocks.append(b)
    return {"tokens": out, "accepts": accepts, "blocks": blocks}


def oracle_draft_fn(cfg, W, mode: str = "mirror") -> DraftFn:
    """Argmax drafts from the oracle drafter (uncached definition)."""
    def fn(blk, pos, valid_from, taps):
        lg = D.draft_block(cfg, W, taps, blk, pos, valid_from, mode)["logits"]
        return D.topk(lg, 1)[0][:, 0]
    return fn
