"""GPU sampling-mode acceptance (dflash_accept_sampled) against the oracle
(oracle/sampling.py):
  - random verify logits over the tiny and the full Qwen3 vocabulary, every
    parameter mix (temperature, top-k, top-p, eps, delta, EOS, budget, block
    lengths 1..8, draft strides 1 and 3), decisions equal to the oracle's
    typical acceptance and card sample, positions and next-round tokens;
  - logits with many exact ties at the k-th value (the index-ordered top-k);
  - eps = 0 (every draft accepted) and the low-temperature limit, which must
    equal the greedy accept of the argmax ids;
  - a sampling-mode round loop of the tiny drafter and the GPU tiny target with
    the adaptive block policy, each round equal to the oracle on the same logits.
Decisions within a relative 1e-5 of the acceptance threshold (the row sums are
fp32 exponentials added in fp64) or whose card sample sits within 1e-12 of a
cumulative boundary are not compared; at least 90% of the cases must be."""
import math

import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from oracle import sampling as S

pytestmark = pytest.mark.gpu


def _binding():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    return binding


def _ambiguous(draft, logits, T, eps, delta, top_k, top_p, seed, rnd, req):
    """True when a rounding-level change could flip the oracle's decision."""
    dl = math.sqrt(eps) if delta is None or delta <= 0 else float(delta)
    acc = len(draft)
    for i, d in enumerate(draft):
        p, H = S.row_stats(logits[i], T)
        thr = min(eps, dl * math.exp(-H))
        if abs(p[d] - thr) <= 1e-5 * max(thr, 1e-300):
            return True
        if not p[d] > thr:
            acc = i
            break
    z = np.asarray(logits[acc], dtype=np.float64)
    order = np.lexsort((np.arange(z.shape[0]), -z))[:top_k]
    x = z[order] / T
    q = np.exp(x - x[0])
    q = q / np.sum(q)
    c = np.cumsum(q)
    u = S.uniform(seed, rnd, req, acc)
    picks = set()
    for tp in (top_p - 1e-12, top_p + 1e-12):
        keep = min(int(np.searchsorted(c, tp, side="left")) + 1, len(order))
        cp = np.cumsum(q[:keep])
        for f in (1 - 1e-12, 1 + 1e-12):
            j = int(np.searchsorted(cp, u * cp[-1] * f, side="right"))
            picks.add(int(order[min(j, keep - 1)]))
    return len(picks) > 1


def _logits(rng, R, b, V, ties=False):
    z = (rng.standard_normal((R, b, V)) * 2.0).astype(np.float32)
    if ties:
        z = (np.round(z * 2.0) / 2.0).astype(np.float32)
    for r in range(R):
        for i in range(b):
            if rng.random() < 0.7:       # a peaked row: one to three tokens well above the rest
                top = rng.choice(V, size=int(rng.integers(1, 4)), replace=False)
                z[r, i, top] += rng.uniform(3.0, 12.0, size=top.shape[0]).astype(np.float32)
    return z


def _drafts(rng, z, k_stride):
    """Drafts [R, b-1, k_stride] (column 0 is the draft): mostly the row's top
    token, else its second token or a random one."""
    R, b, V = z.shape
    d = rng.integers(0, V, (R, max(b - 1, 1), k_stride)).astype(np.int32)
    for r in range(R):
        for i in range(b - 1):
            u = rng.random()
            o = np.argsort(-z[r, i], kind="stable")
            d[r, i, 0] = o[0] if u < 0.6 else o[1] if u < 0.8 else rng.integers(0, V)
    return d


def _compare(dr, cfg, z, d, prm, seed, rnd, eos, budget, p0, what):
    """One dflash_accept_sampled call against the oracle, request by request.
    Returns (compared, excluded)."""
    R, b, V = z.shape
    k_stride = d.shape[2]
    for r in range(R):
        dr.reset(r, 0, p0 + 3 * r)
    zt = torch.from_numpy(z).cuda()
    dt = torch.from_numpy(np.ascontiguousarray(d)).cuda() if b > 1 else None
    bt = None if budget is None else torch.from_numpy(budget).cuda()
    out = dr.accept_sampled(dt, k_stride, zt, temperature=prm["T"], top_k=prm["top_k"], top_p=prm["top_p"],
                            eps=prm["eps"], delta=prm["delta"], seed=seed, round=rnd, eos_id=eos, budget=bt)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in out.items()}
    pos = dr.positions()[0].cpu().numpy()
    comp = excl = 0
    for r in range(R):
        draft = [int(x) for x in d[r, : b - 1, 0]]
        if _ambiguous(draft, z[r], prm["T"], prm["eps"], prm["delta"], prm["top_k"], prm["top_p"], seed, rnd, r):
            excl += 1
            continue
        exp = S.typical_accept(draft, z[r], prm["T"], prm["eps"], prm["delta"], prm["top_k"], prm["top_p"], seed, rnd,
                               r, eos_id=eos, budget=None if budget is None else int(budget[r]))
        ne = exp["n_emit"]
        ctx = (what, r, prm, seed, rnd)
        assert int(o["n_emit"][r]) == ne and int(o["accept_len"][r]) == exp["acc"], (ctx, o["accept_len"][r], exp)
        assert o["emitted"][r, :ne].tolist() == exp["emitted"] and np.all(o["emitted"][r, ne:] == -1), ctx
        assert o["next_tokens"][r].tolist() == D.next_block(exp["emitted"], b, cfg.mask_id), ctx
        assert int(pos[r]) == p0 + 3 * r + ne, ctx
        comp += 1
    return comp, excl


@pytest.mark.parametrize("vocab", [40, 1000, 4096, 151936])
def test_sampled_accept_matches_oracle(vocab):
    """vocab 40 is below the largest top_k (64); 1000 and 151936 end in a
    partial 4096-logit chunk."""
    binding = _binding()
    R = 4
    cfg = config.tiny(max_requests=R).replace(vocab=vocab, mask_id=vocab - 1)
    print(f"case: sampled accept vs oracle, vocab {vocab}", flush=True)
    dr = binding.Drafter(cfg, synth.make_weights(cfg, seed=0, device="cuda"))
    rng = np.random.default_rng(vocab)
    comp = excl = 0
    mixes = [dict(T=1.0, top_k=20, top_p=0.95, eps=0.2, delta=0.0),
             dict(T=0.6, top_k=64, top_p=1.0, eps=0.05, delta=0.0),
             dict(T=1.7, top_k=1, top_p=0.5, eps=0.6, delta=0.3),
             dict(T=1.0, top_k=40, top_p=0.8, eps=0.3, delta=0.9),
             dict(T=0.8, top_k=7, top_p=0.99, eps=0.0, delta=0.0)]
    for trial in range(20):
        prm = mixes[trial % len(mixes)]
        b = [8, 5, 2, 1, 8, 3][trial % 6]
        k_stride = 3 if trial % 4 == 1 else 1
        z = _logits(rng, R, b, vocab, ties=(trial % 5 == 3))
        d = _drafts(rng, z, k_stride)
        eos = int(d[0, 0, 0]) if (trial % 7 == 2 and b > 1) else -1
        budget = rng.integers(0, b + 2, R).astype(np.int32) if trial % 3 == 1 else None
        c, e = _compare(dr, cfg, z, d, prm, seed=1000 + trial, rnd=trial * 3, eos=eos, budget=budget,
                        p0=100 + trial, what=f"trial {trial} b={b}")
        comp += c
        excl += e
    assert dr.check() == 0
    print(f"sampled accept, vocab {vocab}: compared {comp}, near-boundary {excl}", flush=True)
    assert comp >= 0.9 * (comp + excl)


@pytest.mark.parametrize("V", [4096, 20000])
def test_sampled_accept_ties_at_the_kth_value(V):
    """Logits on a coarse grid: many tokens share the k-th value, and the card
    keeps the lowest indices among them (within one 4096-logit chunk, and
    across chunks); flat rows, where every logit ties, take the selection's
    radix path."""
    binding = _binding()
    R, b = 4, 4
    cfg = config.tiny(max_requests=R).replace(vocab=V)
    print(f"case: sampled accept, exact ties at the k-th value, vocab {V}", flush=True)
    dr = binding.Drafter(cfg, synth.make_weights(cfg, seed=0, device="cuda"))
    rng = np.random.default_rng(5)
    comp = excl = 0
    for trial in range(8):
        z = np.floor(rng.standard_normal((R, b, V)) * 1.5).astype(np.float32)
        z[:, :, rng.integers(0, V, 5)] = 9.0          # five tied maxima
        if trial % 4 == 3:
            z[:2] = 0.5                               # flat rows: every logit ties
        d = _drafts(rng, z, 1)
        prm = dict(T=1.0, top_k=[3, 8, 20, 64][trial % 4], top_p=1.0, eps=0.2, delta=0.0)
        c, e = _compare(dr, cfg, z, d, prm, seed=77, rnd=trial, eos=-1, budget=None, p0=10, what=f"ties {trial}")
        comp += c
        excl += e
    print(f"ties: compared {comp}, near-boundary {excl}", flush=True)
    assert comp >= 0.9 * (comp + excl)


def test_sampled_accept_greedy_limit_and_eps_zero():
    binding = _binding()
    R, b, V = 4, 8, 151936
    cfg = config.tiny(max_requests=R).replace(vocab=V)
    print("case: sampled accept at low temperature equals the greedy accept; eps = 0 accepts all", flush=True)
    dr = binding.Drafter(cfg, synth.make_weights(cfg, seed=0, device="cuda"))
    rng = np.random.default_rng(9)
    for trial in range(6):
        z = _logits(rng, R, b, V)
        srt = np.sort(z, axis=2)
        assert np.all(srt[:, :, -1] - srt[:, :, -2] > 0.0)      # no tied argmax
        d = _drafts(rng, z, 1)
        am = np.argmax(z, axis=2).astype(np.int32)
        # greedy limit: T -> 0 with top_k 1 is the argmax; rows whose top two are within 1e-2 are skipped
        if np.all(srt[:, :, -1] - srt[:, :, -2] > 1e-2):
            for r in range(R):
                dr.reset(r, 0, 50)
            zt, dt = torch.from_numpy(z).cuda(), torch.from_numpy(d).cuda()
            s = dr.accept_sampled(dt, 1, zt, temperature=1e-4, top_k=1, top_p=0.95, eps=0.2, seed=trial, round=1)
            for r in range(R):
                dr.reset(r, 0, 50)
            g = dr.accept_n(dt, 1, torch.from_numpy(am).cuda())
            torch.cuda.synchronize()
            for k in ("accept_len", "emitted", "n_emit", "next_tokens"):
                assert torch.equal(s[k], g[k]), (trial, k)
            for r in range(R):
                ref = D.accept(d[r, :, 0].tolist(), am[r].tolist())
                assert int(s["accept_len"][r]) == ref["acc"]
        # eps = 0: every draft with p > 0 is accepted
        for r in range(R):
            dr.reset(r, 0, 50)
        s = dr.accept_sampled(torch.from_numpy(d).cuda(), 1, torch.from_numpy(z).cuda(), temperature=1.0, top_k=20,
                              top_p=0.95, eps=0.0, seed=trial, round=2)
        torch.cuda.synchronize()
        assert torch.all(s["accept_len"] == b - 1) and torch.all(s["n_emit"] == b)
        assert torch.equal(s["emitted"][:, : b - 1].cpu(), torch.from_numpy(d[:, :, 0]))
    assert dr.check() == 0


def test_sampled_accept_refusals():
    binding = _binding()
    cfg = config.tiny(max_requests=2)
    dr = binding.Drafter(cfg, synth.make_weights(cfg, seed=0, device="cuda"))
    z = torch.zeros((2, 4, cfg.vocab), dtype=torch.float32, device="cuda")
    d = torch.zeros((2, 3), dtype=torch.int32, device="cuda")
    for kw in (dict(temperature=0.0), dict(top_k=0), dict(top_k=65), dict(top_p=0.0), dict(top_p=1.5), dict(eps=-1.0)):
        with pytest.raises(binding.DFlashError):
            dr.accept_sampled(d, 1, z, **kw)
    dr.clear_error()
    assert dr.check() == 0


def test_sampling_round_loop_with_block_policy():
    """Tiny drafter + GPU tiny target in sampling mode with the adaptive block
    policy: every round's decision equals the oracle's on the same drafts and
    logits, the policy's block lengths equal the oracle policy's, and the two
    handles' positions track the emitted tokens."""
    binding = _binding()
    dcfg = config.tiny(window=64)
    tcfg = config.tiny(window=128, block=16).replace(n_layers=2)
    wd = synth.make_weights(dcfg, seed=0, device="cuda")
    wt = synth.make_weights(tcfg, seed=11, device="cuda")
    emb = (wd["embed"].float() * 30.0).to(torch.bfloat16)
    wt["embed"], wt["lm_head"] = emb, wd["lm_head"]
    wd["embed"] = emb
    print("case: sampling-mode round loop with the adaptive block policy", flush=True)
    prompt = [5, 17, 300, 4000, 12, 99, 7, 8, 1, 2, 3]
    n_new, B, V = 40, dcfg.block, dcfg.vocab
    # T 0.1: the random-weight tiny target is nearly flat at T 1, where typical
    # acceptance takes any draft; sharpened, wrong drafts are rejected
    prm = dict(T=0.1, top_k=20, top_p=0.95, eps=0.2, delta=0.0)
    seed = 20250
    tg = binding.Drafter(tcfg, wt, target=True)
    dr = binding.Drafter(dcfg, wd)
    tg.reset(0, 0, 0)
    dr.reset(0, 0, len(prompt))
    pos = 0
    while pos < len(prompt):
        chunk = prompt[pos:pos + 16]
        taps = [torch.empty((len(chunk), tcfg.hidden), dtype=torch.float32, device="cuda") for _ in range(2)]
        lg = torch.empty((1, len(chunk), V), dtype=torch.float32, device="cuda")
        tg.verify_block(torch.tensor([chunk], dtype=torch.int32, device="cuda"), [0, 1], taps, lg)
        tg.advance(torch.tensor([len(chunk)], dtype=torch.int32, device="cuda"))
        rows = torch.arange(pos, pos + len(chunk), dtype=torch.int32, device="cuda")
        dr.tap_stage(taps, len(chunk), req_of_row=torch.zeros_like(rows), pos_of_row=rows)
        pos += len(chunk)
    # the first token: a card sample of the prompt's last row (a sampled accept of block length 1)
    first = dr.accept_sampled(None, 1, lg[:, -1:].contiguous(), temperature=prm["T"], top_k=prm["top_k"],
                              top_p=prm["top_p"], eps=prm["eps"], seed=seed, round=0)
    dr.reset(0, 0, len(prompt))
    out = [int(first["emitted"][0, 0])]
    pol, pol_o = binding.BlockPolicy(B), S.BlockPolicy(B)
    blocks, accepts, comp, excl, rnd = [], [], 0, 0, 1
    rng = np.random.default_rng(31)
    while len(out) < n_new:
        b = pol.next_block()
        assert b == pol_o.next_block()
        b = min(b, n_new - len(out) + 1)
        blk = torch.tensor([D.next_block(out, b, dcfg.mask_id)], dtype=torch.int32, device="cuda")
        g_ids = dr.draft_block_n(blk, k=1) if b > 1 else None
        if b > 2 and rnd % 3 != 1:     # most rounds get wrong drafts after the first, so the policy shrinks the block
            g_ids[0, 1:, 0] = torch.from_numpy(rng.integers(0, V - 1, b - 2).astype(np.int32)).cuda()
        draft = g_ids[0, :, 0].cpu().tolist() if b > 1 else []
        vt = torch.tensor([[out[-1]] + draft], dtype=torch.int32, device="cuda")
        taps = [torch.empty((b, tcfg.hidden), dtype=torch.float32, device="cuda") for _ in range(2)]
        lg = torch.empty((1, b, V), dtype=torch.float32, device="cuda")
        tg.verify_block(vt, [0, 1], taps, lg)
        budget = torch.tensor([n_new - len(out)], dtype=torch.int32, device="cuda")
        p_before = len(prompt) + len(out) - 1
        res = dr.accept_sampled(g_ids, 1, lg, temperature=prm["T"], top_k=prm["top_k"], top_p=prm["top_p"],
                                eps=prm["eps"], seed=seed, round=rnd, budget=budget)
        ne, acc = int(res["n_emit"][0]), int(res["accept_len"][0])
        z = lg[0].cpu().numpy()
        if _ambiguous(draft, z, prm["T"], prm["eps"], prm["delta"], prm["top_k"], prm["top_p"], seed, rnd, 0):
            excl += 1
        else:
            exp = S.typical_accept(draft, z, prm["T"], prm["eps"], prm["delta"], prm["top_k"], prm["top_p"], seed, rnd,
                                   0, budget=n_new - len(out))
            assert (acc, ne, res["emitted"][0, :ne].cpu().tolist()) == (exp["acc"], exp["n_emit"], exp["emitted"])
            comp += 1
        tg.advance(res["n_emit"])
        vrows = torch.arange(p_before, p_before + ne, dtype=torch.int32, device="cuda")
        dr.tap_stage([t[:ne] for t in taps], ne, req_of_row=torch.zeros_like(vrows), pos_of_row=vrows)
        out.extend(res["emitted"][0, :ne].cpu().tolist())
        pol.update(acc)
        pol_o.update(acc)
        assert abs(pol.mean - pol_o.mean) < 1e-12
        blocks.append(b)
        accepts.append(acc)
        rnd += 1
        assert int(dr.positions()[0][0]) == int(tg.positions()[0][0]) == len(prompt) + len(out) - 1
    torch.cuda.synchronize()
    assert dr.check() == 0 and tg.check() == 0
    assert len(out) == n_new and all(0 <= t < V for t in out)
    print(f"sampling loop: blocks {blocks}, accepts {accepts}, compared {comp}, near-boundary {excl}", flush=True)
    assert comp >= 0.9 * (comp + excl)
    assert min(blocks) < B            # the policy adapted the block length
