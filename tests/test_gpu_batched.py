"""GPU tests of whole draft/verify loops and of batched requests.

- The lossless loop: the GPU drafter inside the speculative loop against the
  tiny fp64 target must emit exactly the target's greedy continuation, and every
  accept decision must equal the oracle's.
- Batched requests with hyper-connection taps: one call over 8 requests (own
  contexts, positions and lengths) against the oracle per request, and
  bit-exactly against 8 single-request handles (batch invariance).
- The optional ctx RMSNorm after fc.

Everything is called through the C ABI (binding.Drafter)."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from oracle import target as T
from tests import harness as Hn

pytestmark = pytest.mark.gpu


def _binding():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    return binding


def _np(w):
    return {k: ([synth.bf16_to_f32_numpy(t) for t in v] if isinstance(v, list) else synth.bf16_to_f32_numpy(v))
            for k, v in w.items()}


def test_lossless_loop_with_gpu_drafter():
    """Prefill -> (GPU draft -> target verify -> GPU stage of the verify rows ->
    GPU accept) until 40 tokens: output equals greedy decoding of the target."""
    binding = _binding()
    cfg = config.tiny(window=64)
    print("case: lossless loop, tiny drafter on GPU vs tiny fp64 target", flush=True)
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    tcfg = cfg.replace(n_layers=2)
    Wt = _np(synth.make_weights(tcfg, seed=11))
    Wd = _np(wd)
    # a peakier target so greedy continuations vary; the drafter shares its embedding
    Wt["embed"] = Wd["embed"] * 30.0
    Wt["lm_head"] = Wd["lm_head"]
    wd["embed"] = torch.from_numpy(Wt["embed"]).to(torch.bfloat16).cuda()
    tgt = T.TinyTarget(tcfg, Wt, n_layers=2)
    prompt = [5, 17, 300, 4000, 12, 99, 7]
    n_new = 40
    ref = T.greedy(tgt, prompt, n_new)

    dr = binding.Drafter(cfg, wd)
    B = cfg.block
    tgt.reset()
    ids, taps = tgt.feed(prompt, 0)
    pos = len(prompt)
    dr.reset(0, 0, pos)
    rows = torch.arange(0, pos, dtype=torch.int32, device="cuda")
    dr.tap_stage([torch.from_numpy(t).cuda() for t in taps], pos, req_of_row=torch.zeros_like(rows),
                 pos_of_row=rows)
    out = [ids[-1]]
    rounds = 0
    while len(out) < n_new:
        blk = D.next_block(out, B, cfg.mask_id)
        tokens = torch.tensor([blk], dtype=torch.int32, device="cuda")
        g_ids = dr.draft_block(tokens, k=1)
        draft = g_ids[0, :, 0].cpu().tolist()
        verify, vtaps = tgt.feed([blk[0]] + draft, pos)
        vrows = torch.arange(pos, pos + B, dtype=torch.int32, device="cuda")
        dr.tap_stage([torch.from_numpy(t).cuda() for t in vtaps], B, req_of_row=torch.zeros_like(vrows),
                     pos_of_row=vrows)
        budget = torch.tensor([n_new - len(out)], dtype=torch.int32, device="cuda")
        res = dr.accept(g_ids, 1, torch.tensor([verify], dtype=torch.int32, device="cuda"), budget=budget)
        ref_acc = D.accept(draft, verify, eos_id=-1, budget=n_new - len(out))
        n = int(res["n_emit"][0])
        assert n == ref_acc["n_emit"] and int(res["accept_len"][0]) == ref_acc["acc"]
        emitted = res["emitted"][0, :n].cpu().tolist()
        assert emitted == ref_acc["emitted"]
        assert res["next_tokens"][0].cpu().tolist() == D.next_block(out + emitted, B, cfg.mask_id)
        tgt.truncate(pos + n)
        pos += n
        out.extend(emitted)
        rounds += 1
        assert int(dr.positions()[0][0]) == pos
    assert dr.check() == 0
    assert out == ref
    print(f"lossless over {rounds} rounds, {len(out)} tokens", flush=True)


def _stage_requests(dr, cfg, hist, starts, lengths):
    """Stage each request's trailing rows (at most the window) in one call."""
    taps_rows, req, posr = [[] for _ in range(cfg.n_taps)], [], []
    for r, (p0, n) in enumerate(zip(starts, lengths)):
        lo = max(0, n - cfg.window)
        dr.reset(r, p0 - (n - lo), p0)
        for t in range(cfg.n_taps):
            taps_rows[t].append(hist[r][t][lo:n])
        req += [r] * (n - lo)
        posr += list(range(p0 - (n - lo), p0))
    cat = [torch.cat(x, 0).contiguous() for x in taps_rows]
    rq = torch.tensor(req, dtype=torch.int32, device="cuda")
    ps = torch.tensor(posr, dtype=torch.int32, device="cuda")
    dr.tap_stage(cat, len(req), req_of_row=rq, pos_of_row=ps)


def test_hc_batched_requests_tiny():
    """8 requests with 4 hyper-connection streams per tap, different context
    lengths (below and above the window) and positions, in one call: each
    request matches the oracle, and the batch equals single-request calls
    bit for bit."""
    binding = _binding()
    cfg = config.tiny(max_requests=8, hc_streams=4, window=64, max_stage_rows=512)
    print("case: tiny hc=4, 8 requests batched", flush=True)
    w = synth.make_weights(cfg, seed=2, device="cuda")
    wh = Hn.host_weights(w)
    R, B = 8, cfg.block
    lengths = [20, 64, 90, 33, 150, 64, 1, 77]
    starts = [1000 + 37 * r + 5 * lengths[r] for r in range(R)]
    hist = [synth.make_taps(cfg, lengths[r], seed=3, device="cuda", stream=r, outliers=False) for r in range(R)]
    tokens = synth.block_tokens(cfg, R, seed=4, device="cuda")
    dr = binding.Drafter(cfg, w)
    _stage_requests(dr, cfg, hist, starts, lengths)
    logits = torch.empty((R, B - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=16, logits=logits)
    torch.cuda.synchronize()
    assert dr.check() == 0
    g_logits = logits.cpu().numpy()
    g_ids = ids.cpu().numpy()
    for r in range(R):
        n = lengths[r]
        lo = max(0, n - cfg.window)
        taps_h = [np.concatenate([np.zeros((starts[r] - n, t.shape[1])), t.cpu().numpy().astype(np.float64)], 0)
                  for t in hist[r]]
        ref = D.draft_block(cfg, wh, taps_h, tokens[r].cpu().tolist(), starts[r], starts[r] - (n - lo),
                            mode="mirror")
        Hn.assert_close(g_logits[r], ref["logits"], f"request {r} logits")
        Hn.topk_self_consistent(g_logits[r], g_ids[r])
        comp, _ = Hn.topk_agrees_away_from_ties(ref["logits"], g_ids[r], 16, gpu_logits=g_logits[r])
        assert comp > 0
    # batch invariance: the same request alone in its own handle
    one = cfg.replace(max_requests=1)
    for r in range(R):
        d1 = binding.Drafter(one, w)
        _stage_requests(d1, one, [hist[r]], [starts[r]], [lengths[r]])
        l1 = torch.empty((1, B - 1, cfg.vocab), dtype=torch.float32, device="cuda")
        i1 = d1.draft_block(tokens[r:r + 1].contiguous(), k=16, logits=l1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(l1[0].cpu().numpy(), g_logits[r], err_msg=f"request {r} logits")
        np.testing.assert_array_equal(i1[0].cpu().numpy(), g_ids[r], err_msg=f"request {r} ids")


def test_ctx_norm_tiny():
    """ctx_norm = 1: an RMSNorm with its own gain after fc, before the K/V projections."""
    binding = _binding()
    cfg = config.tiny(ctx_norm=1)
    print("case: tiny ctx_norm=1", flush=True)
    w = synth.make_weights(cfg, seed=6, device="cuda")
    wh = Hn.host_weights(w)
    P = 70
    taps = synth.make_taps(cfg, P, seed=7, device="cuda", outliers=True)
    dr = binding.Drafter(cfg, w)
    lo = P - cfg.window
    dr.reset(0, 0, P)
    rows = torch.arange(lo, P, dtype=torch.int32, device="cuda")
    dr.tap_stage([t[lo:] for t in taps], P - lo, req_of_row=torch.zeros_like(rows), pos_of_row=rows)
    tokens = synth.block_tokens(cfg, 1, seed=8, device="cuda")
    logits = torch.empty((1, cfg.block - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=16, logits=logits)
    torch.cuda.synchronize()
    assert dr.check() == 0
    ref = D.draft_block(cfg, wh, [t.cpu().numpy().astype(np.float64) for t in taps], tokens[0].cpu().tolist(), P, 0,
                        mode="mirror", want_intermediates=True)
    Hn.assert_close(logits[0].cpu().numpy(), ref["logits"], "logits")
    rk, rv = dr.ring()
    slots = np.arange(lo, P) % cfg.ring_capacity
    gk = rk[0, 0].float().cpu().numpy()[:, slots, :]
    Hn.assert_close(gk, ref["ctx_k"][0], "ring K")
    Hn.topk_self_consistent(logits[0].cpu().numpy(), ids[0].cpu().numpy())


@pytest.mark.parametrize("W,R", [(512, 8), (1536, 8), (512, 3), (512, 5)])
def test_batch_invariance_qwen3_hc(W, R):
    """qwen3-4b-shaped drafter with 4 hc streams, block 8, R requests with their
    own W-row contexts: a batched round, the stage of the verify rows and the
    accept, then a second batched round, all equal to the same requests run
    alone (bit for bit). Request 0's first round also matches the oracle.
    The batched LM head takes 64 rows (R = 8: four row tiles), 24 (R = 3: two
    tiles, K in phases of 5 chunks) or 40 rows (R = 5: four tiles, the last
    partly padding); each request alone takes the 8-row kernel. At W = 1536 the
    batched attention has 448 (chunk, kv head) workgroups against 112 per
    request alone (query slots split in two), and the combine sums 7 chunk
    partials."""
    binding = _binding()
    cfg = config.qwen3_4b_hc(block=8, window=W, max_requests=R, max_stage_rows=W * R)
    print(f"case: qwen3-4b hc=4 block 8, {R} requests, window {W}", flush=True)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    B = cfg.block
    starts = [W + 37 * r for r in range(R)]   # the oracle indexes taps by absolute position
    hist = [synth.make_taps(cfg, W + 3 * B, seed=9, device="cuda", stream=r, outliers=False) for r in range(R)]
    tokens = synth.block_tokens(cfg, R, seed=10, device="cuda")

    def run(dr, reqs):
        n = len(reqs)
        # prefill: one stage call per request (a call's GEMM plan depends on its
        # row count, so the same call sequence is used with and without batching)
        for i, r in enumerate(reqs):
            dr.reset(i, starts[r] - W, starts[r])
            ps = torch.arange(starts[r] - W, starts[r], dtype=torch.int32, device="cuda")
            dr.tap_stage([hist[r][t][:W] for t in range(cfg.n_taps)], W, req_of_row=torch.full_like(ps, i),
                         pos_of_row=ps)
        lg1 = torch.empty((n, B - 1, cfg.vocab), dtype=torch.float32, device="cuda")
        ids1 = dr.draft_block(tokens[reqs].contiguous(), k=1, logits=lg1)
        # synthetic verify: the draft kept for 2 tokens, then a fixed token
        verify = torch.cat([ids1[:, :2, 0], torch.full((n, B - 2), 7, dtype=torch.int32, device="cuda")], 1)
        vrows = torch.tensor([p for r in reqs for p in range(starts[r], starts[r] + B)], dtype=torch.int32,
                             device="cuda")
        vrq = torch.tensor([i for i in range(n) for _ in range(B)], dtype=torch.int32, device="cuda")
        dr.tap_stage([torch.cat([hist[r][t][W:W + B] for r in reqs], 0).contiguous() for t in range(cfg.n_taps)],
                     n * B, req_of_row=vrq, pos_of_row=vrows)
        res = dr.accept(ids1, 1, verify.contiguous())
        lg2 = torch.empty((n, B - 1, cfg.vocab), dtype=torch.float32, device="cuda")
        ids2 = dr.draft_block(res["next_tokens"], k=16, logits=lg2)
        torch.cuda.synchronize()
        assert dr.check() == 0
        return lg1.cpu().numpy(), ids1.cpu().numpy(), lg2.cpu().numpy(), ids2.cpu().numpy(), \
            res["n_emit"].cpu().numpy()

    batched = run(binding.Drafter(cfg, w), list(range(R)))
    one = cfg.replace(max_requests=1)
    for r in sorted({0, R // 2, R - 1}):
        single = run(binding.Drafter(one, w), [r])
        for a, b, what in zip(batched, single, ("logits 1", "ids 1", "logits 2", "ids 2", "n_emit")):
            np.testing.assert_array_equal(a[r:r + 1], b, err_msg=f"request {r} {what}")
    # request 0, first round, against the oracle (context rows [start-W, start))
    wh = Hn.host_weights(w)
    taps_h = [np.concatenate([np.zeros((starts[0] - W, t.shape[1])), t[:W].cpu().numpy().astype(np.float64)], 0)
              for t in hist[0]]
    ref = D.draft_block(cfg, wh, taps_h, tokens[0].cpu().tolist(), starts[0], starts[0] - W, mode="mirror")
    err = Hn.assert_close(batched[0][0], ref["logits"], "request 0 logits")
    print(f"request 0 logits max err {err:.3g}", flush=True)
