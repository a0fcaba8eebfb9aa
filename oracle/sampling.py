"""Sampling-mode acceptance and the adaptive block-length policy (test
infrastructure only; NumPy, shares no code with the HIP path).

The pages run the drafter with sampling ("dflash: the chain verify builds
pipelined ...", mlx-serve PR #937, "Measured": adaptive block 8 with typical
acceptance 0.2 and card sampling T 1.0, top-p 0.95, top-k 20, a fixed seed;
the round policy of the hyper-connection-stream commit picks the block of each
round). They give no formulas, so this module states them (readings R31-R33 of
the design notes):

R31 typical acceptance. Verify row i gives the target's logits z_i over the
    vocabulary; p_i = softmax(z_i / T), H_i = -sum p_i log p_i. The draft token
    d_i is accepted iff p_i(d_i) > min(eps, delta * exp(-H_i)) (delta =
    sqrt(eps) unless given), the typical-acceptance test of tree/medusa-style
    speculative sampling with eps the pages' "typical 0.2". Acceptance stops at
    the first rejection a (a = B-1 if none); the token after the accepted
    drafts is sampled from the card distribution of row a (R32) with the
    uniform draw of (seed, round, request, a). EOS and budget clamp as in the
    greedy accept.
R32 card sampling. Keep the top_k logits of the row (value desc, index asc),
    q_j = softmax(z_j / T) over them, then the shortest prefix whose q sum
    reaches top_p; the token is the first j of that prefix whose cumulative q
    exceeds u * (sum of the prefix), u in [0, 1).
R33 uniform draws. Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011), key = (seed low 32 bits, seed high
    32 bits), counter = (round, request, row, 0); u = (first output word >> 8) *
    2^-24.
R34 adaptive block policy. Per request an exponential average of the
    accepted drafts, m <- (1 - w) m + w * acc (m starts at block - 1, w = 1/2);
    the next round's block is clamp(floor(m + 1/2) + 2, 2, block): two rows
    beyond the expected accept (rounded to nearest), so a verify pass is not
    wider than the drafter can fill (block itself when block < 2).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(counter: Sequence[int], key: Sequence[int]) -> List[int]:
    """Ten rounds of Philox4x32 on a 4-word counter with a 2-word key."""
    c = [int(x) & MASK for x in counter]
    k0, k1 = int(key[0]) & MASK, int(key[1]) & MASK
    for rnd in range(10):
        if rnd:
            k0, k1 = (k0 + W0) & MASK, (k1 + W1) & MASK
        p0, p1 = M0 * c[0], M1 * c[2]
        c = [((p1 >> 32) ^ c[1] ^ k0) & MASK, p1 & MASK, ((p0 >> 32) ^ c[3] ^ k1) & MASK, p0 & MASK]
    return c


def uniform(seed: int, rnd: int, req: int, row: int) -> float:
    """R33: u in [0, 1) with 24 random bits."""
    w = philox4x32_10([rnd, req, row, 0], [seed & MASK, (seed >> 32) & MASK])
    return (w[0] >> 8) * 2.0 ** -24


def row_stats(z, T: float):
    """(p [V], entropy H) of softmax(z / T) in fp64."""
    x = np.asarray(z, dtype=np.float64) / T
    x = x - np.max(x)
    e = np.exp(x)
    Z = np.sum(e)
    p = e / Z
    H = -float(np.sum(p * (x - math.log(Z))))
    return p, H


def card_sample(z, T: float, top_k: int, top_p: float, u: float) -> int:
    """R32 on one row of logits."""
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(z.shape[0]), -z))[:top_k]
    x = z[order] / T
    q = np.exp(x - x[0])
    q = q / np.sum(q)
    c = np.cumsum(q)
    keep = int(np.searchsorted(c, top_p, side="left")) + 1       # shortest prefix reaching top_p
    keep = min(keep, len(order))
    cp = np.cumsum(q[:keep])
    j = int(np.searchsorted(cp, u * cp[-1], side="right"))       # first j with cumulative > u * total
    return int(order[min(j, keep - 1)])


def typical_accept(draft: Sequence[int], logits, T: float, eps: float, delta: Optional[float], top_k: int,
                   top_p: float, seed: int, rnd: int, req: int, eos_id: int = -1,
                   budget: Optional[int] = None) -> Dict[str, object]:
    """R31 for one request: draft [B-1] ids, logits [B, V] of the verify rows."""
    d = [int(t) for t in draft]
    B = len(d) + 1
    dl = math.sqrt(eps) if delta is None or delta <= 0 else float(delta)
    acc = B - 1
    for i in range(B - 1):
        p, H = row_stats(logits[i], T)
        if not p[d[i]] > min(eps, dl * math.exp(-H)):
            acc = i
            break
    x = card_sample(logits[acc], T, top_k, top_p, uniform(seed, rnd, req, acc))
    emitted = d[:acc] + [x]
    if eos_id >= 0 and eos_id in emitted:
        emitted = emitted[: emitted.index(eos_id) + 1]
    if budget is not None:
        emitted = emitted[: max(int(budget), 1)]
    n = len(emitted)
    return {"acc": min(acc, n - 1), "emitted": emitted, "n_emit": n}


class BlockPolicy:
    """R34 for one request."""

    def __init__(self, block: int, weight: float = 0.5):
        self.block = int(block)
        self.w = float(weight)
        self.mean = float(block - 1)

    def next_block(self) -> int:
        # for block < 2 the range [2, block] is empty: the block itself (target-only rounds)
        return max(min(2, self.block), min(self.block, int(math.floor(self.mean + 0.5)) + 2))

    def update(self, accepted: int):
        self.mean = (1.0 - self.w) * self.mean + self.w * float(accepted)
