"""GPU parity at the benchmark's full sizes (Qwen3-4B-shaped drafter), in the
launch configuration bench.py times: prefill staging of the trailing 4096 rows
of a 16384-row tap buffer, then rounds of draft (top-16) -> verify -> stage ->
accept, each draft compared with the oracle's whole-round recompute."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from tests import harness as Hn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    cfg = config.qwen3_4b(block=16, window=4096, max_stage_rows=4096)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    wh = Hn.host_weights(w)
    return binding, cfg, w, wh


def _check_round(cfg, wh, hist, tokens, pos, vf, logits, ids, what):
    ref = D.draft_block(cfg, wh, hist, tokens, pos, vf, mode="mirror", want_intermediates=True)
    g = logits.cpu().numpy()
    err = float(np.max(np.abs(g - ref["logits"])))
    rms = float(np.sqrt(np.mean((g - ref["logits"]) ** 2)))
    print(f"{what}: logits max err {err:.4g} rms {rms:.3g} (tol {Hn.tol(ref['logits']):.4g}, "
          f"max|oracle| {np.max(np.abs(ref['logits'])):.3g})", flush=True)
    Hn.assert_close(g, ref["logits"], f"{what} logits")
    gi = ids.cpu().numpy()
    Hn.topk_self_consistent(g, gi)
    comp, excl = Hn.topk_agrees_away_from_ties(ref["logits"], gi, gi.shape[-1], gpu_logits=g)
    # top-16: the ranks below the first few sit closer than the error; argmax: most rows decide
    Hn.require_compared(comp, excl, 0.08 if gi.shape[-1] > 1 else 0.40, what)
    worst = Hn.topk_within_eps(ref["logits"], gi, g)
    print(f"{what}: every rank within 2*eps of the oracle's (worst {worst:.2f} of the bound)", flush=True)
    return ref


def test_qwen3_4b_block16_window4096_rounds(big):
    binding, cfg, w, wh = big
    B, V, W = cfg.block, cfg.vocab, cfg.window
    print("case: qwen3-4b-shaped B=16 W=4096 top-16, prefill from a 16384-row buffer", flush=True)
    dr = binding.Drafter(cfg, w)
    total = 16384
    taps = synth.make_taps(cfg, total, seed=0, device="cuda")
    hist = [t.cpu().numpy() for t in taps]
    dr.reset(0, total - W, total)
    dr.tap_stage([t[total - W:] for t in taps], W,
                 req_of_row=torch.zeros(W, dtype=torch.int32, device="cuda"),
                 pos_of_row=torch.arange(total - W, total, dtype=torch.int32, device="cuda"))
    tokens = synth.block_tokens(cfg, 1, seed=0, device="cuda")
    pos, vf = total, total - W
    accepts = [3, 0, 15]
    for rnd in range(3):
        logits = torch.empty((1, B - 1, V), dtype=torch.float32, device="cuda")
        ids = dr.draft_block(tokens, k=16, logits=logits)
        # the call bench.py times: no logits buffer (the head writes its transposed
        # scratch and top-16 reads it back), ids and values only
        ids_b = torch.empty((1, B - 1, 16), dtype=torch.int32, device="cuda")
        vals_b = torch.empty((1, B - 1, 16), dtype=torch.float32, device="cuda")
        dr.draft_block(tokens, k=16, ids=ids_b, vals=vals_b)
        torch.cuda.synchronize()
        assert dr.check() == 0
        np.testing.assert_array_equal(ids_b.cpu().numpy(), ids.cpu().numpy())
        np.testing.assert_array_equal(vals_b[0].cpu().numpy(),
                                      np.take_along_axis(logits[0].cpu().numpy(), ids[0].cpu().numpy(), 1))
        ref = _check_round(cfg, wh, hist, tokens[0].cpu().tolist(), pos, vf, logits[0], ids_b[0], f"round {rnd}")
        if rnd == 0:   # ring contents at sampled window slots equal the oracle's context K/V
            rk, rv = dr.ring()
            sel = np.array([0, 1, 777, 2048, W - 2, W - 1])
            slots = (vf + sel) % cfg.ring_capacity
            for l in (0, cfg.n_layers - 1):
                gk = rk[l, 0].float().cpu().numpy()[:, slots, :]
                gv = rv[l, 0].float().cpu().numpy()[:, :, slots].transpose(0, 2, 1)
                Hn.assert_close(gk, ref["ctx_k"][l][:, sel, :], f"ring K layer {l}")
                Hn.assert_close(gv, ref["ctx_v"][l][:, sel, :], f"ring V layer {l}")
        # synthetic verify with a planted accept length, fresh verify-row taps
        acc = torch.tensor([accepts[rnd]], dtype=torch.int32, device="cuda")
        noise = torch.randint(0, V - 1, (1, B), device="cuda", dtype=torch.int32)
        verify = synth.verify_from_draft(ids[:, :, 0].contiguous(), acc, V, noise)
        vt = synth.make_taps(cfg, B, seed=50 + rnd, device="cuda")
        dr.tap_stage(vt, B, rows_per_req=B)
        out = dr.accept(ids, 16, verify)
        torch.cuda.synchronize()
        exp = D.accept(ids[0, :, 0].cpu().tolist(), verify[0].cpu().tolist())
        n = int(out["n_emit"][0])
        assert int(out["accept_len"][0]) == exp["acc"] == accepts[rnd] and n == exp["n_emit"]
        vt_h = [t.cpu().numpy() for t in vt]
        hist = [np.concatenate([h[:pos], v[:n]], 0) for h, v in zip(hist, vt_h)]
        pos += n
        vf = max(vf, 0)
        assert int(dr.positions()[0][0]) == pos
        tokens = out["next_tokens"]
    assert dr.check() == 0


def test_qwen3_4b_context1024_argmax(big):
    binding, cfg0, w, wh = big
    cfg = cfg0.replace(window=1024, ring_capacity=config.ring_for(1024, 16), max_stage_rows=1024)
    print("case: qwen3-4b-shaped B=16 context 1024 argmax", flush=True)
    dr = binding.Drafter(cfg, w)
    P = 1024
    taps = synth.make_taps(cfg, P, seed=3, device="cuda")
    dr.reset(0, 0, P)
    dr.tap_stage(taps, P, rows_per_req=P, pos_of_row=torch.arange(P, dtype=torch.int32, device="cuda"),
                 req_of_row=torch.zeros(P, dtype=torch.int32, device="cuda"))
    tokens = synth.block_tokens(cfg, 1, seed=4, device="cuda")
    logits = torch.empty((1, cfg.block - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=1, logits=logits)
    torch.cuda.synchronize()
    _check_round(cfg, wh, [t.cpu().numpy() for t in taps], tokens[0].cpu().tolist(), P, 0, logits[0], ids[0],
                 "ctx1024")
    assert dr.check() == 0


def test_hc_eight_requests_window4096_batched():
    """The 8-request workload at its full size, in the launch configuration bench.py
    times: qwen3-4b-shaped drafter fed by 4 hyper-connection streams per tap,
    block 8, every request staging its own 4096-row context window, then one
    batched draft (argmax). Requests 0 and 7 (different start positions, hence
    different chunk alignments) are compared with the oracle's uncached
    recompute of their own windows."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    R, W = 8, 4096
    cfg = config.qwen3_4b(block=8, window=W, max_requests=R, hc_streams=4, max_stage_rows=W)
    B, V = cfg.block, cfg.vocab
    print("case: qwen3-4b hc=4, block 8, 8 requests x 4096-row windows, argmax", flush=True)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    dr = binding.Drafter(cfg, w)
    starts = [W + 37 * r for r in range(R)]
    keep = {}
    for r in range(R):
        taps = synth.make_taps(cfg, W, seed=20, device="cuda", stream=r, outliers=False)
        ps = torch.arange(starts[r] - W, starts[r], dtype=torch.int32, device="cuda")
        dr.reset(r, starts[r] - W, starts[r])
        dr.tap_stage(taps, W, req_of_row=torch.full_like(ps, r), pos_of_row=ps)
        if r in (0, R - 1):
            keep[r] = [t.cpu().numpy() for t in taps]
        del taps
    tokens = synth.block_tokens(cfg, R, seed=21, device="cuda")
    logits = torch.empty((R, B - 1, V), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=1, logits=logits)
    torch.cuda.synchronize()
    assert dr.check() == 0
    wh = Hn.host_weights(w)
    rk, rv = dr.ring()
    for r, th in keep.items():
        # the oracle indexes taps by absolute position: rows before the window are never read
        taps_h = [np.concatenate([np.zeros((starts[r] - W, t.shape[1])), t.astype(np.float64)], 0) for t in th]
        ref = D.draft_block(cfg, wh, taps_h, tokens[r].cpu().tolist(), starts[r], starts[r] - W, mode="mirror",
                            want_intermediates=True)
        # staged context K/V (hc mean + prefill tile path) at sampled window rows
        sel = np.array([0, 1, 1000, 2047, W - 2, W - 1])
        slots = (starts[r] - W + sel) % cfg.ring_capacity
        for l in (0, cfg.n_layers - 1):
            gk = rk[l, r].float().cpu().numpy()[:, slots, :]
            gv = rv[l, r].float().cpu().numpy()[:, :, slots].transpose(0, 2, 1)
            ek = Hn.assert_close(gk, ref["ctx_k"][l][:, sel, :], f"request {r} ring K layer {l}")
            ev = Hn.assert_close(gv, ref["ctx_v"][l][:, sel, :], f"request {r} ring V layer {l}")
            print(f"request {r} layer {l}: ring K err {ek:.3g} (tol {Hn.tol(ref['ctx_k'][l][:, sel, :]):.3g}), "
                  f"V err {ev:.3g} (tol {Hn.tol(ref['ctx_v'][l][:, sel, :]):.3g})", flush=True)
        g = logits[r].cpu().numpy()
        t = Hn.tol(ref["logits"])
        err = Hn.assert_close(g, ref["logits"], f"request {r} logits")
        rms = float(np.sqrt(np.mean((g - ref["logits"]) ** 2)))
        print(f"request {r}: logits max err {err:.4g} rms {rms:.3g}, tol {t:.4g} (max|oracle| "
              f"{np.max(np.abs(ref['logits'])):.3g}), {err / t:.0%} of the tolerance", flush=True)
        comp, excl = Hn.topk_agrees_away_from_ties(ref["logits"], ids[r].cpu().numpy(), 1, gpu_logits=g)
        Hn.require_compared(comp, excl, 0.40, f"request {r} argmax")
        Hn.topk_within_eps(ref["logits"], ids[r].cpu().numpy(), g)


def test_qwen3_4b_block8_window4096_top16(big):
    """The block-8 workload at its full size: the same drafter, one request, the
    trailing 4096 rows of a 16384-row tap buffer staged, one draft of 7 mask rows
    with top-16, against the oracle."""
    binding, cfg0, w, wh = big
    cfg = cfg0.replace(block=8, ring_capacity=config.ring_for(4096, 8))
    B, V, W = cfg.block, cfg.vocab, cfg.window
    print("case: qwen3-4b-shaped B=8 W=4096 top-16, prefill from a 16384-row buffer", flush=True)
    dr = binding.Drafter(cfg, w)
    total = 16384
    taps = synth.make_taps(cfg, total, seed=11, device="cuda")
    dr.reset(0, total - W, total)
    dr.tap_stage([t[total - W:] for t in taps], W,
                 req_of_row=torch.zeros(W, dtype=torch.int32, device="cuda"),
                 pos_of_row=torch.arange(total - W, total, dtype=torch.int32, device="cuda"))
    tokens = synth.block_tokens(cfg, 1, seed=12, device="cuda")
    logits = torch.empty((1, B - 1, V), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=16, logits=logits)
    torch.cuda.synchronize()
    assert dr.check() == 0
    hist = [t.cpu().numpy() for t in taps]
    _check_round(cfg, wh, hist, tokens[0].cpu().tolist(), total, total - W, logits[0], ids[0], "block 8")
