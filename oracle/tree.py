"""Candidate trees from the drafter's top-k lists, tree-masked verify and tree
acceptance (test infrastructure only; fp64 NumPy, shares no code with the HIP
path).

The pages keep top-16 candidates per draft position and hand them to a path
selector ("feat: DFlash2 block-diffusion drafter for Qwen 3.8", Mference PR #22,
"What's here" and the Metal-port commit: "top-16 + CPU path selector"), and
mention a tree verify round beside the chain verify ("dflash: the chain verify
builds pipelined ...", mlx-serve PR #937). Neither page gives the selection
rule or the tree layout, so this module states one (readings R28-R30 of the
design notes):

R28 candidate tree. Node 0 is the root: the block's known token at position
    pos. A node at depth d (1 <= d <= B-1) holds one of the top-k candidates
    of draft position d; its children are the k candidates of position d+1
    (block diffusion drafts every position from the same masked block, so the
    candidate lists do not depend on the parent). Within the list of position
    d, candidate j has log-probability
        lp_d[j] = (v_d[j] - v_d[0]) - log(sum_j' exp(v_d[j'] - v_d[0]))
    (the softmax of the top-k logits; differences and sums in fp64, j' in list
    order), and a node's score is the sum of lp along its path, added in depth
    order. The tree of n nodes is: the root; the top-1 chain (rank 0 at every
    depth, up to depth min(B-1, n-1)); then, best first, the highest-scoring
    child of any node already in the tree until n nodes are chosen. Ties go to
    the smaller depth, then the smaller parent index, then the smaller rank.
    Nodes are numbered in the order chosen, so a parent precedes its children.
R29 tree verify. The target runs every node as one row at position
    pos + depth, attending to the committed context and to the node's own
    ancestors (itself included): each node's result is the target's greedy
    next token after the root path leading to it.
R30 tree accept. Walk from the root: while the current node has a child whose
    token equals the target's token at the current node, move there (children
    hold distinct tokens). Emitted = the tokens of the walked path after the
    root, then the target's token at the last node reached (the bonus). EOS
    and budget clamp as in the chain accept; the committed rows are the first
    n_emit nodes of the walked path (the root first), and pos += n_emit. A
    tree that is just the chain accepts exactly as the chain rule does.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import dflash as D


def list_logprobs(vals) -> np.ndarray:
    """lp[d][j] of R28 for values [D][k] (fp32 logits sorted descending per row)."""
    v = np.asarray(vals, dtype=np.float64)
    out = np.empty_like(v)
    for d in range(v.shape[0]):
        gaps = v[d] - v[d][0]
        s = 0.0
        for g in gaps:               # list order
            s += math.exp(g)
        out[d] = gaps - math.log(s)
    return out


def build_tree(root: int, ids, vals, n_nodes: int) -> Dict[str, List]:
    """The candidate tree of R28 from top-k ids/values [B-1][k] of one request.
    Returns tokens, parent (-1 for the root), depth, rank (-1 for the root) and
    score per node, in node order."""
    ids = np.asarray(ids)
    Dm, k = ids.shape
    lp = list_logprobs(vals)
    tokens, parent, depth, rank, score = [int(root)], [-1], [0], [-1], [0.0]
    taken = set()                    # (parent, rank) pairs in the tree
    # the top-1 chain
    while len(tokens) < n_nodes and depth[-1] < Dm:
        p = len(tokens) - 1
        d = depth[p] + 1
        tokens.append(int(ids[d - 1][0]))
        parent.append(p)
        depth.append(d)
        rank.append(0)
        score.append(score[p] + lp[d - 1][0])
        taken.add((p, 0))
    # best first over every child of a node in the tree
    while len(tokens) < n_nodes:
        best = None
        for p in range(len(tokens)):
            d = depth[p] + 1
            if d > Dm:
                continue
            for j in range(k):
                if (p, j) in taken:
                    continue
                key = (-(score[p] + lp[d - 1][j]), d, p, j)
                if best is None or key < best:
                    best = key
        if best is None:
            break
        _, d, p, j = best
        tokens.append(int(ids[d - 1][j]))
        parent.append(p)
        depth.append(d)
        rank.append(j)
        score.append(score[p] + lp[d - 1][j])
        taken.add((p, j))
    return {"tokens": tokens, "parent": parent, "depth": depth, "rank": rank, "score": score}


def ancestors(parent: Sequence[int]) -> List[set]:
    """Ancestor sets (each node included) from a parent array in node order."""
    out = []
    for i, p in enumerate(parent):
        out.append({i} | (out[p] if p >= 0 else set()))
    return out


def root_path(parent: Sequence[int], i: int) -> List[int]:
    path = []
    while i >= 0:
        path.append(i)
        i = parent[i]
    return path[::-1]


def tree_accept(tokens: Sequence[int], parent: Sequence[int], verify: Sequence[int], block: int,
                eos_id: int = -1, budget: Optional[int] = None) -> Dict[str, object]:
    """R30 for one request: tokens/parent of the tree, verify[i] = the target's
    token at node i. Returns acc (depth reached, after the clamps), emitted,
    n_emit and path (the committed nodes, root first, n_emit of them)."""
    n = len(tokens)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    cur, path = 0, [0]
    while True:
        nxt = [c for c in children[cur] if tokens[c] == verify[cur]]
        assert len(nxt) <= 1, "children must hold distinct tokens"
        if not nxt:
            break
        cur = nxt[0]
        path.append(cur)
    acc = len(path) - 1
    emitted = [int(tokens[i]) for i in path[1:]] + [int(verify[cur])]
    assert len(emitted) <= block
    if eos_id >= 0 and eos_id in emitted:
        emitted = emitted[: emitted.index(eos_id) + 1]
    if budget is not None:
        emitted = emitted[: max(int(budget), 1)]
    n_emit = len(emitted)
    return {"acc": min(acc, n_emit - 1), "emitted": emitted, "n_emit": n_emit, "path": path[:n_emit]}


def speculative_tree(target, draft_lists, prompt: Sequence[int], n_new: int, block: int, n_nodes: int,
                     mask_id: int, eos_id: int = -1) -> Dict[str, object]:
    """The tree round loop against a TinyTarget: draft top-k lists -> tree (R28)
    -> tree verify (R29, each node's greedy token) -> tree accept (R30) ->
    commit the walked path's rows. ``draft_lists(block_tokens, pos, taps)``
    returns (ids [B-1][k], vals [B-1][k]); taps[t] holds the committed tap rows
    [0, pos). Returns the emitted tokens and per-round accept depths."""
    target.reset()
    ids0, taps = target.feed(prompt, 0)
    committed = [t.copy() for t in taps]
    pos = len(prompt)
    out = [ids0[-1]]
    accepts = []
    while len(out) < n_new and out[-1] != eos_id:
        blk = D.next_block(out, block, mask_id)
        ids, vals = draft_lists(blk, pos, committed)
        tree = build_tree(blk[0], ids, vals, n_nodes)
        verify, node_taps = tree_verify(target, tree["tokens"], tree["parent"], pos)
        res = tree_accept(tree["tokens"], tree["parent"], verify, block, eos_id=eos_id, budget=n_new - len(out))
        rows = [tree["tokens"][i] for i in res["path"]]
        _, ctaps = target.feed(rows, pos)            # the committed rows enter the cache
        for t in range(len(committed)):
            committed[t] = np.concatenate([committed[t], ctaps[t]], 0)
            assert np.array_equal(ctaps[t], node_taps[t][res["path"]])
        pos += res["n_emit"]
        out.extend(res["emitted"])
        accepts.append(res["acc"])
    return {"tokens": out, "accepts": accepts}


def tree_verify(target, tokens: Sequence[int], parent: Sequence[int], pos: int):
    """R29 with a TinyTarget whose cache holds positions [0, pos): each node's
    greedy token and its tap rows, every node fed as the last row of its root
    path (the cache is left as it was). Returns (verify [n], taps [L][n, H])."""
    verify, rows = [], []
    for i in range(len(tokens)):
        path = root_path(parent, i)
        ids, taps = target.feed([tokens[j] for j in path], pos)
        target.truncate(pos)
        verify.append(int(ids[-1]))
        rows.append([t[-1] for t in taps])
    L = len(rows[0])
    return verify, [np.stack([r[l] for r in rows], 0) for l in range(L)]
