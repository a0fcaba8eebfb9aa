"""GPU parity of the draft round (tiny drafter) against the fp64 oracle.

Everything is called through the C ABI (binding.Drafter). Inputs come from
synth on the GPU and are copied to the host for the oracle."""
import ctypes

import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from tests import harness as Hn

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    return binding


@pytest.fixture(scope="module")
def tiny_setup():
    binding = _gpu()
    cfg = config.tiny(max_requests=4)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    wh = Hn.host_weights(w)
    return binding, cfg, w, wh


def _taps_history(cfg, n, seed):
    taps = synth.make_taps(cfg, n, seed=seed, device="cuda", outliers=True)
    return taps, [t.cpu().numpy().astype(np.float64) for t in taps]


def test_single_round_parity_tiny(tiny_setup):
    binding, cfg, w, wh = tiny_setup
    print(f"case: tiny single round B={cfg.block} W={cfg.window} C={cfg.ring_capacity}", flush=True)
    dr = binding.Drafter(cfg, w)
    P = 100
    taps, taps_h = _taps_history(cfg, P, seed=0)
    lo = P - cfg.window
    dr.reset(0, 0, P)
    rows = torch.arange(lo, P, dtype=torch.int32, device="cuda")
    dr.tap_stage([t[lo:] for t in taps], P - lo, req_of_row=torch.zeros_like(rows), pos_of_row=rows)
    tokens = synth.block_tokens(cfg, 1, seed=0, device="cuda")
    logits = torch.empty((1, cfg.block - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    vals = torch.empty((1, cfg.block - 1, 16), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=16, logits=logits, vals=vals)
    ids1 = dr.draft_block(tokens, k=1)
    torch.cuda.synchronize()
    assert dr.check() == 0

    ref = D.draft_block(cfg, wh, taps_h, tokens[0].cpu().tolist(), P, 0, mode="mirror", want_intermediates=True)
    g_logits = logits[0].cpu().numpy()
    err = Hn.assert_close(g_logits, ref["logits"], "logits")
    exact = D.draft_block(cfg, wh, taps_h, tokens[0].cpu().tolist(), P, 0, mode="exact")
    print(f"logits max err {err:.3g} (mirror); oracle mirror-vs-exact drift "
          f"{np.max(np.abs(ref['logits'] - exact['logits'])):.3g}", flush=True)
    g_ids = ids.cpu().numpy()
    Hn.topk_self_consistent(g_logits, g_ids[0])
    np.testing.assert_array_equal(vals[0].cpu().numpy(), np.take_along_axis(g_logits, g_ids[0], 1))
    np.testing.assert_array_equal(ids1.cpu().numpy()[0, :, 0], g_ids[0, :, 0])
    comp, excl = Hn.topk_agrees_away_from_ties(ref["logits"], g_ids[0], 16, gpu_logits=g_logits)
    print(f"top-16 ranks compared {comp}, excluded as near-ties {excl}", flush=True)
    assert comp > 0

    # the ring holds the oracle's context K/V (cached == uncached)
    rk, rv = dr.ring()
    slots = np.arange(lo, P) % cfg.ring_capacity
    for l in range(cfg.n_layers):
        gk = rk[l, 0].float().cpu().numpy()[:, slots, :]                 # [nkv, n, hd]
        gv = rv[l, 0].float().cpu().numpy()[:, :, slots].transpose(0, 2, 1)
        Hn.assert_close(gk, ref["ctx_k"][l], f"ring K layer {l}")
        Hn.assert_close(gv, ref["ctx_v"][l], f"ring V layer {l}")


def test_short_context_and_reset_tiny(tiny_setup):
    """Context shorter than the window, and context length 0 after a reset."""
    binding, cfg, w, wh = tiny_setup
    dr = binding.Drafter(cfg, w)
    taps, taps_h = _taps_history(cfg, 40, seed=1)
    tokens = synth.block_tokens(cfg, 1, seed=3, device="cuda")
    for P, vf in ((20, 0), (37, 37), (40, 33)):
        print(f"case: tiny pos={P} valid_from={vf}", flush=True)
        dr.reset(0, vf, P)
        if P > vf:
            dr.tap_stage([t[vf:] for t in taps], P - vf, rows_per_req=P - vf,
                         pos_of_row=torch.arange(vf, P, dtype=torch.int32, device="cuda"),
                         req_of_row=torch.zeros(P - vf, dtype=torch.int32, device="cuda"))
        logits = torch.empty((1, cfg.block - 1, cfg.vocab), dtype=torch.float32, device="cuda")
        dr.draft_block(tokens, k=1, logits=logits)
        torch.cuda.synchronize()
        ref = D.draft_block(cfg, wh, taps_h, tokens[0].cpu().tolist(), P, vf, mode="mirror")
        Hn.assert_close(logits[0].cpu().numpy(), ref["logits"], f"logits pos={P} vf={vf}")
    assert dr.check() == 0


def test_rounds_with_accept_and_rollback_tiny(tiny_setup):
    """Many rounds: draft -> synthetic verify -> stage verify rows -> accept.
    Verify rows carry fresh taps every round (a rejected row's taps differ from
    the one later committed at that position), the ring wraps, and every draft
    must equal the oracle recomputing the context from the committed taps."""
    binding, cfg, w, wh = tiny_setup
    dr = binding.Drafter(cfg, w)
    B, V = cfg.block, cfg.vocab
    P0 = 70
    pre, pre_h = _taps_history(cfg, P0, seed=5)
    history = [h.copy() for h in pre_h]
    lo = max(0, P0 - cfg.window)
    dr.reset(0, 0, P0)
    dr.tap_stage([t[lo:] for t in pre], P0 - lo, rows_per_req=1,
                 pos_of_row=torch.arange(lo, P0, dtype=torch.int32, device="cuda"),
                 req_of_row=torch.zeros(P0 - lo, dtype=torch.int32, device="cuda"))
    tokens = synth.block_tokens(cfg, 1, seed=7, device="cuda")
    accepts = synth.geometric_accepts(12, 1, B, p=0.75, seed=1)
    gen = torch.Generator(device="cuda").manual_seed(9)
    pos = P0
    for rnd in range(12):
        print(f"case: tiny round {rnd} pos={pos}", flush=True)
        logits = torch.empty((1, B - 1, V), dtype=torch.float32, device="cuda")
        ids = dr.draft_block(tokens, k=1, logits=logits)
        torch.cuda.synchronize()
        ref = D.draft_block(cfg, wh, history, tokens[0].cpu().tolist(), pos, 0, mode="mirror")
        Hn.assert_close(logits[0].cpu().numpy(), ref["logits"], f"round {rnd} logits")
        noise = torch.randint(0, V - 1, (1, B), generator=gen, device="cuda", dtype=torch.int32)
        acc = torch.tensor(accepts[rnd], dtype=torch.int32, device="cuda")
        verify = synth.verify_from_draft(ids[:, :, 0].contiguous(), acc, V, noise)
        vt = synth.make_taps(cfg, B, seed=100 + rnd, device="cuda")
        dr.tap_stage(vt, B, rows_per_req=B)             # rows at [pos, pos + B)
        out = dr.accept(ids, 1, verify)
        torch.cuda.synchronize()
        exp = D.accept(ids[0, :, 0].cpu().tolist(), verify[0].cpu().tolist())
        assert int(out["accept_len"][0]) == exp["acc"] == int(accepts[rnd, 0])
        n = int(out["n_emit"][0])
        assert n == exp["n_emit"]
        assert out["emitted"][0, :n].cpu().tolist() == exp["emitted"]
        vt_h = [t.cpu().numpy().astype(np.float64) for t in vt]
        history = [np.concatenate([h[:pos], v[:n]], 0) for h, v in zip(history, vt_h)]
        pos += n
        assert int(dr.positions()[0][0]) == pos
        nt = out["next_tokens"][0].cpu().tolist()
        assert nt == D.next_block(exp["emitted"], B, cfg.mask_id)
        tokens = out["next_tokens"]
    st = dr.stats().cpu().numpy()
    assert st[0] == 12 and st[B + 1] == pos - P0
    for i in range(B):
        assert st[1 + i] == int(np.sum(accepts[:12, 0] > i))
    assert dr.check() == 0


def test_accept_kernel_cases(tiny_setup):
    binding, cfg, w, wh = tiny_setup
    dr = binding.Drafter(cfg, w)
    B, R = cfg.block, 4
    rng = np.random.default_rng(0)
    for trial in range(40):
        d = rng.integers(0, 5, (R, B - 1)).astype(np.int32)
        v = rng.integers(0, 5, (R, B)).astype(np.int32)
        for r in range(R):                       # plant matching prefixes
            a = rng.integers(0, B)
            v[r, :a] = d[r, :a] if a < B else v[r, :a]
        eos = int(rng.integers(-1, 5)) if trial % 3 else -1
        budget = rng.integers(-1, B + 2, R).astype(np.int32) if trial % 2 else None
        for r in range(R):
            dr.reset(r, 0, 1000 + r)
        out = dr.accept(torch.from_numpy(d).cuda(), 1, torch.from_numpy(v).cuda(), eos_id=eos,
                        budget=None if budget is None else torch.from_numpy(budget).cuda())
        torch.cuda.synchronize()
        pos = dr.positions()[0].cpu().numpy()
        for r in range(R):
            exp = D.accept(d[r].tolist(), v[r].tolist(), eos_id=eos,
                           budget=None if budget is None else int(budget[r]))
            n = exp["n_emit"]
            assert int(out["accept_len"][r]) == exp["acc"]
            assert int(out["n_emit"][r]) == n
            em = out["emitted"][r].cpu().tolist()
            assert em[:n] == exp["emitted"] and all(x == -1 for x in em[n:])
            assert pos[r] == 1000 + r + n
            assert out["next_tokens"][r].cpu().tolist() == D.next_block(exp["emitted"], B, cfg.mask_id)


def test_topk_exact_ties_tiny(tiny_setup):
    """Massive exact ties in the logits: the LM head's rows repeat with period 37,
    so every logit value occurs ~110 times. Top-16 and argmax must still be the
    (value desc, index asc) order of the GPU's own logits, bit-exact."""
    binding, cfg, w, wh = tiny_setup
    print("case: tiny top-k with repeated LM-head rows", flush=True)
    w2 = dict(w)
    period = 37
    base = w["lm_head"][:period]
    w2["lm_head"] = base.repeat((cfg.vocab + period - 1) // period, 1)[:cfg.vocab].contiguous()
    dr = binding.Drafter(cfg, w2)
    P = 40
    taps, _ = _taps_history(cfg, P, seed=5)
    dr.reset(0, 0, P)
    rows = torch.arange(0, P, dtype=torch.int32, device="cuda")
    dr.tap_stage([t[:P] for t in taps], P, req_of_row=torch.zeros_like(rows), pos_of_row=rows)
    tokens = synth.block_tokens(cfg, 1, seed=3, device="cuda")
    logits = torch.empty((1, cfg.block - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    vals = torch.empty((1, cfg.block - 1, 16), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=16, logits=logits, vals=vals)
    ids1 = dr.draft_block(tokens, k=1)
    torch.cuda.synchronize()
    assert dr.check() == 0
    g_logits = logits[0].cpu().numpy()
    g_ids = ids.cpu().numpy()[0]
    # ties really are there: the best value repeats in every row
    assert all(np.sum(g_logits[r] == g_logits[r].max()) > 16 for r in range(g_logits.shape[0]))
    Hn.topk_self_consistent(g_logits, g_ids)
    np.testing.assert_array_equal(vals[0].cpu().numpy(), np.take_along_axis(g_logits, g_ids, 1))
    np.testing.assert_array_equal(ids1.cpu().numpy()[0, :, 0], g_ids[:, 0])


@pytest.mark.parametrize("V", [128, 200])
def test_topk_vocab_below_k_groups_tiny(tiny_setup, V):
    """A vocabulary of fewer 16-column groups than k (8 and 13 groups for k 16):
    every candidate is ranked, so the top-16 is still the stable sort of the
    GPU's own logits, in the caller's layout and in the transposed scratch."""
    binding, cfg0, _, _ = tiny_setup
    cfg = cfg0.replace(vocab=V, mask_id=V - 1)
    print(f"case: tiny top-16 with vocab {V}", flush=True)
    w = synth.make_weights(cfg, seed=4, device="cuda")
    wh = Hn.host_weights(w)
    dr = binding.Drafter(cfg, w)
    P = 60
    taps, taps_h = _taps_history(cfg, P, seed=6)
    dr.reset(0, 0, P)
    rows = torch.arange(0, P, dtype=torch.int32, device="cuda")
    dr.tap_stage([t[:P] for t in taps], P, req_of_row=torch.zeros_like(rows), pos_of_row=rows)
    tokens = synth.block_tokens(cfg, 1, seed=2, device="cuda")
    logits = torch.empty((1, cfg.block - 1, V), dtype=torch.float32, device="cuda")
    vals = torch.empty((1, cfg.block - 1, 16), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=16, logits=logits, vals=vals)
    vals_t = torch.empty((1, cfg.block - 1, 16), dtype=torch.float32, device="cuda")
    ids_t = dr.draft_block(tokens, k=16, vals=vals_t)   # no caller logits: the transposed scratch
    torch.cuda.synchronize()
    assert dr.check() == 0
    g_logits = logits[0].cpu().numpy()
    g_ids = ids.cpu().numpy()[0]
    Hn.topk_self_consistent(g_logits, g_ids)
    np.testing.assert_array_equal(vals[0].cpu().numpy(), np.take_along_axis(g_logits, g_ids, 1))
    np.testing.assert_array_equal(ids_t.cpu().numpy()[0], g_ids)
    np.testing.assert_array_equal(vals_t.cpu().numpy()[0], vals[0].cpu().numpy())
    ref = D.draft_block(cfg, wh, taps_h, tokens[0].cpu().tolist(), P, 0, mode="mirror")
    Hn.assert_close(g_logits, ref["logits"], "logits")
    comp, excl = Hn.topk_agrees_away_from_ties(ref["logits"], g_ids, 16, gpu_logits=g_logits)
    print(f"top-16 ranks compared {comp}, excluded as near-ties {excl}", flush=True)
    assert comp > 0


def test_empty_and_oversized_calls_refused_before_any_launch(tiny_setup):
    """Host validation on a bound handle: a staging call of 0 rows or of more rows
    than the workspace holds, a draft of 0 or too many requests, a block length of
    0 or above the configured block, k outside {1, 16}, and an accept of 0 or too
    many requests are each refused with their status before anything is enqueued:
    positions, the ring and the device error word are unchanged afterwards, and
    the handle still drafts."""
    binding, cfg, w, _ = tiny_setup
    E_ARG, E_SHAPE, E_CAPACITY = -1, -3, -4
    dr = binding.Drafter(cfg, w)
    P, B = 20, cfg.block
    taps = synth.make_taps(cfg, P, seed=5, device="cuda")
    dr.reset(0, 0, P)
    dr.tap_stage(taps, P, req_of_row=torch.zeros(P, dtype=torch.int32, device="cuda"),
                 pos_of_row=torch.arange(P, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    pos0 = [t.clone() for t in dr.positions()]
    ring0 = [t.clone() for t in dr.ring()]
    tokens = synth.block_tokens(cfg, cfg.max_requests + 1, seed=6, device="cuda")
    ids = torch.empty((cfg.max_requests + 1, B, 16), dtype=torch.int32, device="cuda")
    verify = torch.ones((cfg.max_requests + 1, B), dtype=torch.int32, device="cuda")

    # the wrappers check shapes before the C ABI (ValueError); these calls go
    # straight through the C ABI so that its own checks decide, with live buffers
    lib, ctx, st = dr.lib, dr.ctx, binding._stream()
    Rx = cfg.max_requests + 1
    tp = (ctypes.c_void_p * cfg.n_taps)(*[t.data_ptr() for t in taps])
    tpp = ctypes.cast(tp, binding.PP)
    out = {"accept_len": torch.empty(Rx, dtype=torch.int32, device="cuda"),
           "emitted": torch.empty((Rx, B), dtype=torch.int32, device="cuda"),
           "n_emit": torch.empty(Rx, dtype=torch.int32, device="cuda"),
           "next_tokens": torch.empty((Rx, B), dtype=torch.int32, device="cuda")}

    def acc(n):
        return lib.dflash_accept(ctx, st, ids.data_ptr(), 16, verify.data_ptr(), n, -1, None,
                                 out["accept_len"].data_ptr(), out["emitted"].data_ptr(), out["n_emit"].data_ptr(),
                                 out["next_tokens"].data_ptr())

    cases = [
        ("stage of 0 rows", E_SHAPE, lambda: lib.dflash_tap_stage(ctx, st, tpp, taps[0].stride(0), 0, None, None, 1)),
        ("stage beyond max_stage_rows", E_CAPACITY,
         lambda: lib.dflash_tap_stage(ctx, st, tpp, taps[0].stride(0), cfg.max_stage_rows + 1, None, None, 1)),
        ("draft of 0 requests", E_SHAPE,
         lambda: lib.dflash_draft_block(ctx, st, tokens.data_ptr(), 0, None, ids.data_ptr(), None, 1)),
        ("block length 0", E_SHAPE,
         lambda: lib.dflash_draft_block_n(ctx, st, tokens.data_ptr(), 1, 0, None, ids.data_ptr(), None, 1)),
        ("draft with a null token pointer", E_ARG,
         lambda: lib.dflash_draft_block(ctx, st, None, 1, None, ids.data_ptr(), None, 1)),
        ("draft beyond max_requests", E_SHAPE,
         lambda: lib.dflash_draft_block(ctx, st, tokens.data_ptr(), Rx, None, ids.data_ptr(), None, 1)),
        ("block length above the block", E_SHAPE,
         lambda: lib.dflash_draft_block_n(ctx, st, tokens.data_ptr(), 1, B + 1, None, ids.data_ptr(), None, 1)),
        ("k = 3", E_ARG, lambda: lib.dflash_draft_block(ctx, st, tokens.data_ptr(), 1, None, ids.data_ptr(), None, 3)),
        ("accept of 0 requests", E_SHAPE, lambda: acc(0)),
        ("accept beyond max_requests", E_SHAPE, lambda: acc(Rx)),
    ]
    for what, code, fn in cases:
        rc = fn()
        assert rc == code, (what, rc, binding.last_error())
        print(f"{what}: {binding.STATUS[rc]}: {binding.last_error()}", flush=True)
    torch.cuda.synchronize()
    for a, b in zip(dr.positions(), pos0):
        assert torch.equal(a, b)
    for a, b in zip(dr.ring(), ring0):
        assert torch.equal(a, b)
    assert dr.check() == 0
    got = dr.draft_block(tokens[:1].contiguous(), k=1)
    torch.cuda.synchronize()
    assert dr.check() == 0 and got.shape == (1, B - 1, 1)


def _stage_rows(dr, taps, positions):
    """Stage the tap rows of the given absolute positions (request 0)."""
    pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
    rows = [t[pos.long()].contiguous() for t in taps]
    dr.tap_stage(rows, len(positions), req_of_row=torch.zeros_like(pos), pos_of_row=pos)


def test_ring_capacity_guard_tiny(tiny_setup):
    """A staged row whose ring slot holds another live row of its request (the
    live positions are the window and the block, [pos - W, pos + B)) is skipped
    and sets DFLASH_DEV_RING_CAPACITY: the ring is left bit for bit as it was,
    valid rows of the same call are still written, and after the error is
    cleared the next draft equals the oracle. Checked on the few-row (split-K)
    staging path and on the prefill (tiled) path."""
    binding, cfg, w, wh = tiny_setup
    B, W, C = cfg.block, cfg.window, cfg.ring_capacity
    P = 300
    taps, taps_h = _taps_history(cfg, P + 200, seed=13)
    tokens = synth.block_tokens(cfg, 1, seed=14, device="cuda")
    RING_CAPACITY = 16
    hi, lo = P + C - W, P + B - C - 1            # first positions past either end of the rule
    print(f"case: ring capacity guard, pos={P} W={W} B={B} C={C}: valid [{lo + 1}, {hi})", flush=True)

    # few rows: two bad rows around one valid row (slot of position P - W - 1, outside the window)
    dr = binding.Drafter(cfg, w)
    dr.reset(0, P - W, P)
    _stage_rows(dr, taps, list(range(P - W, P)))
    torch.cuda.synchronize()
    assert dr.check() == 0
    before = [t.clone() for t in dr.ring()]
    _stage_rows(dr, taps, [hi, hi - 1, lo])
    torch.cuda.synchronize()
    word = dr.check()
    assert word == RING_CAPACITY, hex(word)
    after = dr.ring()
    ok_slot = (hi - 1) % C
    keep = np.ones(C, dtype=bool)
    keep[ok_slot] = False
    for b, a, name in ((before[0], after[0], "K"), (before[1], after[1], "V")):
        bb, aa = b.cpu(), a.cpu()
        sl = (slice(None), slice(None), slice(None), torch.from_numpy(keep)) if name == "K" else \
             (slice(None), slice(None), slice(None), slice(None), torch.from_numpy(keep))
        assert torch.equal(bb[sl], aa[sl]), f"ring {name} changed outside the valid row's slot"
    assert not torch.equal(before[0][:, 0, :, ok_slot], after[0][:, 0, :, ok_slot]), "the valid row was not written"
    dr.clear_error()
    logits = torch.empty((1, B - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    dr.draft_block(tokens, k=1, logits=logits)
    torch.cuda.synchronize()
    assert dr.check() == 0
    ref = D.draft_block(cfg, wh, taps_h, tokens[0].cpu().tolist(), P, P - W, mode="mirror")
    Hn.assert_close(logits[0].cpu().numpy(), ref["logits"], "draft after the refused rows")

    # the prefill path (>= 256 rows): the window staged four times over, then again
    # with one row moved to a position past the upper end
    n = 4 * W
    assert n >= 256 and n <= cfg.max_stage_rows
    dr2 = binding.Drafter(cfg, w)
    dr2.reset(0, P - W, P)
    rows = [P - W + (i % W) for i in range(n)]
    _stage_rows(dr2, taps, rows)
    torch.cuda.synchronize()
    assert dr2.check() == 0
    before = [t.clone() for t in dr2.ring()]
    rows[5] = hi + 3
    _stage_rows(dr2, taps, rows)
    torch.cuda.synchronize()
    word = dr2.check()
    assert word == RING_CAPACITY, hex(word)
    for b, a in zip(before, dr2.ring()):
        assert torch.equal(b, a), "the prefill path wrote a refused row or changed the window"
