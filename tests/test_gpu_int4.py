"""GPU parity of the INT4-projection drafter (symmetric INT4, groups of 64,
fp16 scales) against the fp64 oracle run on the exact dequantized weights.

The tiny case covers the split-K GEMM with the X slice staged in LDS (draft and
per-round staging, layer-batched stage K/V). The Qwen3-8B-shaped case runs the
workload's own sizes: a 2048-row prefill (one workgroup per column group and row
chunk over the whole K range, X fragments read from L2 for fc's 20480-wide
input), then rounds at block 8 with staging and accept, and a block-6 handle."""
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


def _check(cfg, wq, hist, tokens, pos, vf, logits, ids, what):
    ref = D.draft_block(cfg, wq, hist, tokens, pos, vf, mode="mirror", want_intermediates=True)
    g = logits.cpu().numpy()
    err = Hn.assert_close(g, ref["logits"], f"{what} logits")
    gi = ids.cpu().numpy()
    Hn.topk_self_consistent(g, gi)
    comp, excl = Hn.topk_agrees_away_from_ties(ref["logits"], gi, gi.shape[-1], gpu_logits=g)
    print(f"{what}: logits max err {err:.4g} (tol {Hn.tol(ref['logits']):.4g}); "
          f"top-k ranks compared {comp}, near-ties excluded {excl}", flush=True)
    assert comp > 0
    return ref


def test_int4_rounds_tiny():
    binding = _gpu()
    cfg = config.tiny(wfmt=config.WFMT_INT4_G64)
    print(f"case: tiny INT4 B={cfg.block} W={cfg.window}", flush=True)
    w = synth.make_weights(cfg, seed=5, device="cuda")
    wq = D.dequantize(Hn.host_weights(w))
    dr = binding.Drafter(cfg, w)
    P = 90
    taps = synth.make_taps(cfg, P, seed=6, device="cuda", outliers=True)
    hist = [t.cpu().numpy() for t in taps]
    lo = P - cfg.window
    dr.reset(0, lo, P)
    dr.tap_stage([t[lo:] for t in taps], P - lo, req_of_row=torch.zeros(P - lo, dtype=torch.int32, device="cuda"),
                 pos_of_row=torch.arange(lo, P, dtype=torch.int32, device="cuda"))
    tokens = synth.block_tokens(cfg, 1, seed=7, device="cuda")
    pos, vf, B, V = P, lo, cfg.block, cfg.vocab
    for rnd, acc_len in enumerate([2, 7, 0]):
        logits = torch.empty((1, B - 1, V), dtype=torch.float32, device="cuda")
        ids = dr.draft_block(tokens, k=16, logits=logits)
        torch.cuda.synchronize()
        assert dr.check() == 0
        ref = _check(cfg, wq, hist, tokens[0].cpu().tolist(), pos, vf, logits[0], ids[0], f"tiny int4 round {rnd}")
        if rnd == 0:
            rk, rv = dr.ring()
            slots = np.arange(vf, pos) % cfg.ring_capacity
            gk = rk[0, 0].float().cpu().numpy()[:, slots, :]
            gv = rv[0, 0].float().cpu().numpy()[:, :, slots].transpose(0, 2, 1)
            Hn.assert_close(gk, ref["ctx_k"][0], "ring K")
            Hn.assert_close(gv, ref["ctx_v"][0], "ring V")
        acc = torch.tensor([acc_len], dtype=torch.int32, device="cuda")
        noise = torch.randint(0, V - 1, (1, B), device="cuda", dtype=torch.int32)
        verify = synth.verify_from_draft(ids[:, :, 0].contiguous(), acc, V, noise)
        vt = synth.make_taps(cfg, B, seed=60 + rnd, device="cuda")
        dr.tap_stage(vt, B, rows_per_req=B)
        out = dr.accept(ids, 16, verify)
        torch.cuda.synchronize()
        n = int(out["n_emit"][0])
        assert int(out["accept_len"][0]) == acc_len and n == acc_len + 1
        hist = [np.concatenate([h[:pos], v.cpu().numpy()[:n]], 0) for h, v in zip(hist, vt)]
        pos += n
        tokens = out["next_tokens"]
    assert dr.check() == 0


def test_int4_qwen3_8b_prefill_and_rounds():
    binding = _gpu()
    cfg = config.qwen3_8b_int4(block=8, window=2048, max_stage_rows=2048)
    print("case: qwen3-8b-shaped INT4 B=8 W=2048, prefill 2048 rows of a 4096-row buffer", flush=True)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    wq = D.dequantize(Hn.host_weights(w))
    total, W, B, V = 4096, cfg.window, cfg.block, cfg.vocab
    taps = synth.make_taps(cfg, total, seed=1, device="cuda")
    hist = [t.cpu().numpy() for t in taps]
    dr = binding.Drafter(cfg, w)
    dr.reset(0, total - W, total)
    dr.tap_stage([t[total - W:] for t in taps], W, req_of_row=torch.zeros(W, dtype=torch.int32, device="cuda"),
                 pos_of_row=torch.arange(total - W, total, dtype=torch.int32, device="cuda"))
    tokens = synth.block_tokens(cfg, 1, seed=2, device="cuda")
    pos, vf = total, total - W
    for rnd, acc_len in enumerate([4, 1]):
        logits = torch.empty((1, B - 1, V), dtype=torch.float32, device="cuda")
        ids = dr.draft_block(tokens, k=16, logits=logits)
        ids1 = dr.draft_block(tokens, k=1)
        torch.cuda.synchronize()
        assert dr.check() == 0
        _check(cfg, wq, hist, tokens[0].cpu().tolist(), pos, vf, logits[0], ids[0], f"8b int4 round {rnd}")
        np.testing.assert_array_equal(ids1[0, :, 0].cpu().numpy(), ids[0, :, 0].cpu().numpy())
        acc = torch.tensor([acc_len], dtype=torch.int32, device="cuda")
        noise = torch.randint(0, V - 1, (1, B), device="cuda", dtype=torch.int32)
        verify = synth.verify_from_draft(ids[:, :, 0].contiguous(), acc, V, noise)
        vt = synth.make_taps(cfg, B, seed=70 + rnd, device="cuda")
        dr.tap_stage(vt, B, rows_per_req=B)
        out = dr.accept(ids, 16, verify)
        torch.cuda.synchronize()
        n = int(out["n_emit"][0])
        assert int(out["accept_len"][0]) == acc_len and n == acc_len + 1
        hist = [np.concatenate([h[:pos], v.cpu().numpy()[:n]], 0) for h, v in zip(hist, vt)]
        pos += n
        vf = max(vf, pos - W)
        assert int(dr.positions()[0][0]) == pos
        tokens = out["next_tokens"]
    # block 6 with the same weights: a fresh handle over the last 2048 rows
    cfg6 = cfg.replace(block=6, ring_capacity=config.ring_for(W, 6))
    dr6 = binding.Drafter(cfg6, w)
    dr6.reset(0, pos - W, pos)
    hist_t = [torch.from_numpy(h[pos - W:pos]).to("cuda") for h in hist]
    dr6.tap_stage(hist_t, W, req_of_row=torch.zeros(W, dtype=torch.int32, device="cuda"),
                  pos_of_row=torch.arange(pos - W, pos, dtype=torch.int32, device="cuda"))
    tok6 = synth.block_tokens(cfg6, 1, seed=3, device="cuda")
    logits6 = torch.empty((1, 5, V), dtype=torch.float32, device="cuda")
    ids6 = dr6.draft_block(tok6, k=16, logits=logits6)
    torch.cuda.synchronize()
    assert dr6.check() == 0
    _check(cfg6, wq, hist, tok6[0].cpu().tolist(), pos, pos - W, logits6[0], ids6[0], "8b int4 block 6")


def test_int4_batch_invariance_qwen3_8b():
    """Qwen3-8B-shaped INT4 drafter, block 8: two requests drafted in one call
    (16 rows: the split-K INT4 gate/up and its SiLU finish) equal each request
    drafted alone (8 rows: the one-launch INT4 gate/up), logits and top-16 bit
    for bit. The single-request path is the one the oracle test above covers."""
    binding = _gpu()
    W = 256
    cfg = config.qwen3_8b_int4(block=8, window=W, max_requests=2, max_stage_rows=2 * W)
    print("case: qwen3-8b-shaped INT4 B=8 W=256, 2 requests batched vs alone", flush=True)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    R, B, V = 2, cfg.block, cfg.vocab
    starts = [W + 29 * r for r in range(R)]
    hist = [synth.make_taps(cfg, W, seed=11, device="cuda", stream=r) for r in range(R)]
    tokens = synth.block_tokens(cfg, R, seed=12, device="cuda")

    def run(dr, reqs):
        # one stage call per request, so that both runs use the same GEMM plans
        for i, r in enumerate(reqs):
            dr.reset(i, starts[r] - W, starts[r])
            ps = torch.arange(starts[r] - W, starts[r], dtype=torch.int32, device="cuda")
            dr.tap_stage([hist[r][t] for t in range(cfg.n_taps)], W, req_of_row=torch.full_like(ps, i),
                         pos_of_row=ps)
        lg = torch.empty((len(reqs), B - 1, V), dtype=torch.float32, device="cuda")
        ids = dr.draft_block(tokens[reqs].contiguous(), k=16, logits=lg)
        torch.cuda.synchronize()
        assert dr.check() == 0
        return lg.cpu().numpy(), ids.cpu().numpy()

    batched = run(binding.Drafter(cfg, w), [0, 1])
    one = cfg.replace(max_requests=1)
    for r in range(R):
        single = run(binding.Drafter(one, w), [r])
        np.testing.assert_array_equal(batched[0][r:r + 1], single[0], err_msg=f"request {r} logits")
        np.testing.assert_array_equal(batched[1][r:r + 1], single[1], err_msg=f"request {r} top-16")
    print("batched == alone for both requests", flush=True)
