"""GPU candidate trees against the oracle (oracle/tree.py):
  - dflash_tree_build on the drafter's own top-16 lists and on synthetic lists,
    bit-exact against the oracle's best-first tree;
  - dflash_tree_accept, bit-exact against the oracle's walk (EOS, budget, the
    staging rows and positions, the drafter's positions);
  - dflash_verify_tree on the tiny causal target against the oracle target fed
    each node's root path (logits, argmax away from ties, taps);
  - the whole tree loop on the GPU (draft top-16 -> tree -> tree verify ->
    tree accept -> target commit -> staging of the committed rows) equal to the
    GPU target's own greedy decoding, with the drafter's lists and with planted
    lists that hold the target's token at a random rank."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from oracle import target as T
from oracle import tree as TR
from tests import harness as Hn

pytestmark = pytest.mark.gpu


def _binding():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    return binding


def _synthetic_lists(rng, R, Dm, k, V):
    ids = np.stack([np.stack([rng.choice(V, size=k, replace=False) for _ in range(Dm)]) for _ in range(R)])
    vals = -np.sort(-rng.standard_normal((R, Dm, k)).astype(np.float32), axis=2)
    return ids.astype(np.int32), vals


def _gpu_tree_vs_oracle(dr, tokens, ids, vals, n, what):
    tok, par, dep = dr.tree_build(tokens, ids, vals, n)
    torch.cuda.synchronize()
    tok, par, dep = tok.cpu().numpy(), par.cpu().numpy(), dep.cpu().numpy()
    for r in range(tokens.shape[0]):
        ref = TR.build_tree(int(tokens[r, 0]), ids[r].cpu().numpy(), vals[r].cpu().numpy(), n)
        assert tok[r].tolist() == ref["tokens"], (what, r, n)
        assert par[r].tolist() == ref["parent"], (what, r, n)
        assert dep[r].tolist() == ref["depth"], (what, r, n)
    return tok, par, dep


def test_tree_build_matches_oracle_tiny():
    binding = _binding()
    cfg = config.tiny(max_requests=3)
    print("case: tree build, drafter top-16 lists and synthetic lists", flush=True)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    dr = binding.Drafter(cfg, w)
    R, B = 3, cfg.block
    for r in range(R):
        taps = synth.make_taps(cfg, 70, seed=40, device="cuda", stream=r)
        rows = torch.arange(6, 70, dtype=torch.int32, device="cuda")
        dr.reset(r, 6, 70)
        dr.tap_stage([t[6:] for t in taps], 64, req_of_row=torch.full_like(rows, r), pos_of_row=rows)
    tokens = synth.block_tokens(cfg, R, seed=41, device="cuda")
    ids = torch.empty((R, B - 1, 16), dtype=torch.int32, device="cuda")
    vals = torch.empty((R, B - 1, 16), dtype=torch.float32, device="cuda")
    dr.draft_block(tokens, k=16, ids=ids, vals=vals)
    for n in (1, 5, 8, 16, 33, 64):
        _gpu_tree_vs_oracle(dr, tokens, ids, vals, n, "drafter lists")
    rng = np.random.default_rng(42)
    for k in (16, 4, 1):
        si, sv = _synthetic_lists(rng, R, B - 1, k, cfg.vocab)
        si_t, sv_t = torch.from_numpy(si).cuda(), torch.from_numpy(sv).cuda()
        for n in ((1, 8) if k == 1 else (2, 8, 20, 64)):
            _gpu_tree_vs_oracle(dr, tokens, si_t, sv_t, n, f"synthetic k={k}")
    # exact ties: every candidate of a list has the same value
    sv0 = torch.zeros_like(sv_t)
    _gpu_tree_vs_oracle(dr, tokens, si_t, sv0, 8, "all ties k=1")
    si16, _ = _synthetic_lists(rng, R, B - 1, 16, cfg.vocab)
    _gpu_tree_vs_oracle(dr, tokens, torch.from_numpy(si16).cuda(),
                        torch.zeros((R, B - 1, 16), dtype=torch.float32, device="cuda"), 40, "all ties k=16")
    assert dr.check() == 0


def test_tree_accept_matches_oracle_tiny():
    binding = _binding()
    cfg = config.tiny(max_requests=4)
    print("case: tree accept vs the oracle walk (EOS, budget)", flush=True)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    dr = binding.Drafter(cfg, w)
    R, B, n = 4, cfg.block, 24
    rng = np.random.default_rng(43)
    for trial in range(30):
        si, sv = _synthetic_lists(rng, R, B - 1, 16, 50)
        roots = rng.integers(0, 50, R)
        trees = [TR.build_tree(int(roots[r]), si[r], sv[r], n) for r in range(R)]
        verify = np.zeros((R, n), dtype=np.int32)
        for r in range(R):
            # the target's continuation: the listed rank-0 w.p. .5, another listed rank w.p. .4, else unlisted
            g = [int(si[r, d, 0]) if (u := rng.random()) < 0.5 else int(si[r, d, rng.integers(1, 16)]) if u < 0.9
                 else 60 + d for d in range(B - 1)] + [77]
            verify[r] = [g[trees[r]["depth"][i]] if rng.random() < 0.9 else int(rng.integers(0, 50)) for i in range(n)]
        eos = int(rng.integers(-1, 50)) if trial % 3 else -1
        budget = rng.integers(0, B + 2, R).astype(np.int32) if trial % 2 else None
        for r in range(R):
            dr.reset(r, 0, 500 + 7 * r)
        tok = torch.tensor([t["tokens"] for t in trees], dtype=torch.int32, device="cuda")
        par = torch.tensor([t["parent"] for t in trees], dtype=torch.int32, device="cuda")
        out = dr.tree_accept(tok, par, torch.from_numpy(verify).cuda(), eos_id=eos,
                             budget=None if budget is None else torch.from_numpy(budget).cuda())
        torch.cuda.synchronize()
        pos = dr.positions()[0].cpu().numpy()
        o = {k_: v.cpu().numpy() for k_, v in out.items()}
        for r in range(R):
            exp = TR.tree_accept(trees[r]["tokens"], trees[r]["parent"], verify[r].tolist(), B, eos_id=eos,
                                 budget=None if budget is None else int(budget[r]))
            ne = exp["n_emit"]
            assert int(o["n_emit"][r]) == ne and int(o["accept_len"][r]) == exp["acc"], (trial, r)
            assert o["emitted"][r, :ne].tolist() == exp["emitted"] and np.all(o["emitted"][r, ne:] == -1)
            assert o["path_nodes"][r, :ne].tolist() == exp["path"]
            assert o["stage_rows"][r, :ne].tolist() == [r * n + i for i in exp["path"]]
            assert o["stage_pos"][r].tolist() == [500 + 7 * r + d for d in range(B)]
            assert o["next_tokens"][r].tolist() == D.next_block(exp["emitted"], B, cfg.mask_id)
            assert int(pos[r]) == 500 + 7 * r + ne
    assert dr.check() == 0


def _pair(target_block=16):
    binding = _binding()
    dcfg = config.tiny(window=64)
    tcfg = config.tiny(window=128, block=target_block).replace(n_layers=2)
    wd = synth.make_weights(dcfg, seed=0, device="cuda")
    wt = synth.make_weights(tcfg, seed=11, device="cuda")
    emb = (wd["embed"].float() * 30.0).to(torch.bfloat16)
    wt["embed"], wt["lm_head"] = emb, wd["lm_head"]
    wd["embed"] = emb
    return binding, dcfg, tcfg, wd, wt


def _np(w):
    return {k: ([synth.bf16_to_f32_numpy(t) for t in v] if isinstance(v, list) else synth.bf16_to_f32_numpy(v))
            for k, v in w.items()}


def test_verify_tree_vs_oracle_target_tiny():
    binding, dcfg, tcfg, wd, wt = _pair()
    print("case: tree verify (16 nodes) on the tiny target vs the oracle target", flush=True)
    tg = binding.Drafter(tcfg, wt, target=True)
    tg.reset(0, 0, 0)
    prompt = [5, 17, 300, 4000, 12, 99, 7, 8, 1, 2, 3, 4, 55, 66, 77, 88, 9, 10, 11]
    for c0 in range(0, len(prompt), 16):
        chunk = prompt[c0:c0 + 16]
        tg.verify_block(torch.tensor([chunk], dtype=torch.int32, device="cuda"))
        tg.advance(torch.tensor([len(chunk)], dtype=torch.int32, device="cuda"))
    P = len(prompt)
    rng = np.random.default_rng(44)
    si, sv = _synthetic_lists(rng, 1, dcfg.block - 1, 16, dcfg.vocab)
    tree = TR.build_tree(33, si[0], sv[0], 16)
    n = 16
    tok = torch.tensor([tree["tokens"]], dtype=torch.int32, device="cuda")
    par = torch.tensor([tree["parent"]], dtype=torch.int32, device="cuda")
    dep = torch.tensor([tree["depth"]], dtype=torch.int32, device="cuda")
    taps = [torch.empty((n, tcfg.hidden), dtype=torch.float32, device="cuda") for _ in range(2)]
    logits = torch.empty((1, n, tcfg.vocab), dtype=torch.float32, device="cuda")
    ids = tg.verify_tree(tok, par, dep, [0, 1], taps, logits)
    torch.cuda.synchronize()
    assert tg.check() == 0
    assert int(tg.positions()[0][0]) == P          # a verify pass does not move pos
    ref = T.TinyTarget(tcfg, _np(wt), n_layers=2, mode="mirror")
    ref.feed(prompt, 0)
    verify_o, taps_o = TR.tree_verify(ref, tree["tokens"], tree["parent"], P)
    rows = []
    for i in range(n):       # each node's logits: the last row of its root path fed after the prompt
        rows.append(ref.feed([tree["tokens"][j] for j in TR.root_path(tree["parent"], i)], P, want_logits=True)[2][-1])
        ref.truncate(P)
    lg_o = np.stack(rows)
    g = logits[0].cpu().numpy()
    err = Hn.assert_close(g, lg_o, "tree verify logits")
    comp, excl = Hn.topk_agrees_away_from_ties(lg_o, ids.cpu().numpy().reshape(-1, 1), 1, gpu_logits=g)
    Hn.require_compared(comp, excl, 0.5, "tree verify argmax")
    ga = ids[0].cpu().numpy()
    sure = [i for i in range(n) if np.sort(lg_o[i])[-1] - np.sort(lg_o[i])[-2] > 2 * float(np.max(np.abs(g[i] - lg_o[i])))]
    assert all(int(ga[i]) == verify_o[i] for i in sure)
    for l in range(2):
        Hn.assert_close(taps[l].cpu().numpy(), taps_o[l], f"tree verify taps layer {l}")
    print(f"tree verify: logits err {err:.3g}, argmax compared {comp}, near-ties {excl}", flush=True)


@pytest.mark.parametrize("lists", ["drafter", "planted"])
def test_tree_loop_lossless_tiny(lists):
    """The tree round loop on the GPU emits the GPU target's greedy decoding."""
    binding, dcfg, tcfg, wd, wt = _pair()
    print(f"case: GPU tree loop ({lists} lists, 16 nodes) vs GPU target greedy", flush=True)
    prompt = [5, 17, 300, 4000, 12, 99, 7, 8, 1, 2, 3]
    n_new, n, B, V = 40, 16, dcfg.block, dcfg.vocab
    rng = np.random.default_rng(45)

    def prefill(tg, dr):
        pos, last = 0, None
        while pos < len(prompt):
            chunk = prompt[pos:pos + 16]
            taps = [torch.empty((len(chunk), tcfg.hidden), dtype=torch.float32, device="cuda") for _ in range(2)]
            ids = tg.verify_block(torch.tensor([chunk], dtype=torch.int32, device="cuda"), [0, 1], taps)
            tg.advance(torch.tensor([len(chunk)], dtype=torch.int32, device="cuda"))
            if dr is not None:
                rows = torch.arange(pos, pos + len(chunk), dtype=torch.int32, device="cuda")
                dr.tap_stage(taps, len(chunk), req_of_row=torch.zeros_like(rows), pos_of_row=rows)
            pos += len(chunk)
            last = ids
        return [int(last[0, -1])]

    tg = binding.Drafter(tcfg, wt, target=True)
    tg.reset(0, 0, 0)
    ref = prefill(tg, None)
    while len(ref) < n_new + B:
        ids = tg.verify_block(torch.tensor([[ref[-1]]], dtype=torch.int32, device="cuda"))
        tg.advance(torch.tensor([1], dtype=torch.int32, device="cuda"))
        ref.append(int(ids[0, 0]))

    tg = binding.Drafter(tcfg, wt, target=True)
    dr = binding.Drafter(dcfg, wd)
    tg.reset(0, 0, 0)
    dr.reset(0, 0, len(prompt))
    out = prefill(tg, dr)
    accepts, chain_accepts = [], []
    d_ids = torch.empty((1, B - 1, 16), dtype=torch.int32, device="cuda")
    d_vals = torch.empty((1, B - 1, 16), dtype=torch.float32, device="cuda")
    while len(out) < n_new:
        blk = torch.tensor([D.next_block(out, B, dcfg.mask_id)], dtype=torch.int32, device="cuda")
        dr.draft_block(blk, k=16, ids=d_ids, vals=d_vals)
        if lists == "planted":
            start = len(out)
            pi = np.stack([rng.permutation(V - 1)[:16] for _ in range(B - 1)]).astype(np.int32)
            ranks = []
            for d in range(B - 1):
                true = ref[start + d] if start + d < len(ref) else 0
                pi[d] = [x if x != true else (x + 1) % (V - 1) for x in pi[d]]
                rk = int(rng.integers(0, 5))
                if rk < 4:
                    pi[d][rk] = true
                ranks.append(rk)
            # what the top-1 chain alone would accept: the leading positions holding the target's token at rank 0
            chain_accepts.append(next((d for d, rk in enumerate(ranks) if rk != 0), B - 1))
            pv = -np.sort(-rng.standard_normal((B - 1, 16)).astype(np.float32), axis=1)
            d_ids.copy_(torch.from_numpy(pi).view(1, B - 1, 16))
            d_vals.copy_(torch.from_numpy(pv).view(1, B - 1, 16))
        tok, par, dep = dr.tree_build(blk, d_ids, d_vals, n)
        taps = [torch.empty((n, tcfg.hidden), dtype=torch.float32, device="cuda") for _ in range(2)]
        v_ids = tg.verify_tree(tok, par, dep, [0, 1], taps)
        budget = torch.tensor([n_new - len(out)], dtype=torch.int32, device="cuda")
        res = dr.tree_accept(tok, par, v_ids, budget=budget)
        tg.tree_commit(res["path_nodes"], res["n_emit"])
        dr.tap_stage_rows(taps, res["stage_rows"].view(-1), res["stage_pos"].view(-1), rows_per_req=B)
        ne = int(res["n_emit"][0])
        out.extend(res["emitted"][0, :ne].cpu().tolist())
        accepts.append(int(res["accept_len"][0]))
        assert int(dr.positions()[0][0]) == int(tg.positions()[0][0]) == len(prompt) + len(out) - 1
    torch.cuda.synchronize()
    assert dr.check() == 0 and tg.check() == 0
    assert out == ref[:n_new], (out, ref[:n_new])
    print(f"tree loop: {len(accepts)} rounds, accepts {accepts}", flush=True)
    if lists == "planted":
        # the budget can cut the last round short; every other round accepts at least what the chain would
        assert all(a >= c for a, c in zip(accepts[:-1], chain_accepts[:-1]))
        assert sum(accepts) > sum(chain_accepts)
        print(f"chain alone would accept {chain_accepts}", flush=True)


def test_tree_verify_fullsize_vs_oracle_target():
    """A 16-node tree pass at the qwen3-4b layer shape (hidden 2560, 32/8 heads x
    128, ffn 9728, vocab 151936; 4 layers, window 4096) after a 300-row prompt,
    against the mirror oracle target walking the tree depth first: each node is
    one row at pos + depth over the prompt and the node's ancestors (logits,
    argmax away from ties, the taps after layers 1 and 3)."""
    binding = _binding()
    tcfg = config.qwen3_4b(block=16, window=4096, max_stage_rows=16).replace(n_layers=4)
    V, H, P, n = tcfg.vocab, tcfg.hidden, 300, 16
    print("case: qwen3-4b-shaped 4-layer target, prompt 300, 16-node tree from block-8 lists", flush=True)
    wt = synth.make_weights(tcfg, seed=21, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(23)
    prompt = torch.randint(0, V - 1, (P,), generator=g, device="cuda", dtype=torch.int32).cpu().tolist()
    tg = binding.Drafter(tcfg, wt, target=True)
    tg.reset(0, 0, 0)
    for r0 in range(0, P, 16):
        chunk = prompt[r0:r0 + 16]
        tg.verify_block(torch.tensor([chunk], dtype=torch.int32, device="cuda"))
        tg.advance(torch.tensor([len(chunk)], dtype=torch.int32, device="cuda"))
    rng = np.random.default_rng(24)
    si, sv = _synthetic_lists(rng, 1, 7, 16, V - 1)
    tree = TR.build_tree(int(rng.integers(0, V - 1)), si[0], sv[0], n)
    tok = torch.tensor([tree["tokens"]], dtype=torch.int32, device="cuda")
    par = torch.tensor([tree["parent"]], dtype=torch.int32, device="cuda")
    dep = torch.tensor([tree["depth"]], dtype=torch.int32, device="cuda")
    taps = [torch.empty((n, H), dtype=torch.float32, device="cuda") for _ in range(2)]
    logits = torch.empty((1, n, V), dtype=torch.float32, device="cuda")
    ids = tg.verify_tree(tok, par, dep, [1, 3], taps, logits)
    torch.cuda.synchronize()
    assert tg.check() == 0
    assert int(tg.positions()[0][0]) == P
    ref = T.TinyTarget(tcfg, _np(wt), n_layers=4, mode="mirror")
    ref.prefill(prompt)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[tree["parent"][i]].append(i)
    lg_o = np.zeros((n, V))
    taps_o = [np.zeros((n, H), dtype=np.float32) for _ in range(2)]
    stack = [0]
    while stack:                       # depth first: the cache holds the prompt and the node's ancestors
        v = stack.pop()
        d = tree["depth"][v]
        ref.truncate(P + d)
        _, tr, lg = ref.feed([tree["tokens"][v]], P + d, want_logits=True)
        lg_o[v] = lg[0]
        taps_o[0][v], taps_o[1][v] = tr[1][0], tr[3][0]
        stack.extend(reversed(children[v]))
    gl = logits[0].cpu().numpy()
    err = Hn.assert_close(gl, lg_o, "tree verify logits (full size)")
    comp, excl = Hn.topk_agrees_away_from_ties(lg_o, ids.cpu().numpy().reshape(-1, 1), 1, gpu_logits=gl)
    Hn.require_compared(comp, excl, 0.5, "tree verify argmax (full size)")
    et = [Hn.assert_close(taps[i].cpu().numpy(), taps_o[i], f"tree tap after layer {l}") for i, l in enumerate((1, 3))]
    print(f"full-size tree verify: logits err {err:.3g}, tap errs {et[0]:.3g} {et[1]:.3g}, argmax compared {comp}, "
          f"near-ties {excl}", flush=True)
