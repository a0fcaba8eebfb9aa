"""GPU parity of prefill staging: a staging call of at least 256 rows takes the
tap-gather + tiled-GEMM path. Checked against the oracle (ring K/V and a draft
round) on the tiny drafter with ragged row tiles, one and four hyper-connection
streams, with and without the context RMSNorm, bf16 and INT4 weights; and
against the same rows staged by the split-K path in chunks below the threshold."""
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


@pytest.mark.parametrize("hc,ctx_norm,wfmt", [(1, 0, config.WFMT_BF16), (4, 0, config.WFMT_BF16),
                                               (1, 1, config.WFMT_BF16), (1, 0, config.WFMT_INT4_G64)])
def test_prefill_tiny_vs_oracle(hc, ctx_norm, wfmt):
    binding = _gpu()
    W, P = 300, 340
    cfg = config.tiny(window=W, max_stage_rows=600, hc_streams=hc, ctx_norm=ctx_norm, wfmt=wfmt)
    print(f"case: tiny prefill hc={hc} ctx_norm={ctx_norm} wfmt={wfmt} rows={W}", flush=True)
    w = synth.make_weights(cfg, seed=3, device="cuda")
    wh = D.dequantize(Hn.host_weights(w))
    taps = synth.make_taps(cfg, P, seed=4, device="cuda", outliers=(hc == 1))
    hist = [t.cpu().numpy() for t in taps]
    dr = binding.Drafter(cfg, w)
    lo = P - W
    dr.reset(0, lo, P)
    dr.tap_stage([t[lo:] for t in taps], W, req_of_row=torch.zeros(W, dtype=torch.int32, device="cuda"),
                 pos_of_row=torch.arange(lo, P, dtype=torch.int32, device="cuda"))
    tokens = synth.block_tokens(cfg, 1, seed=5, device="cuda")
    logits = torch.empty((1, cfg.block - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    ids = dr.draft_block(tokens, k=16, logits=logits)
    torch.cuda.synchronize()
    assert dr.check() == 0
    ref = D.draft_block(cfg, wh, hist, tokens[0].cpu().tolist(), P, lo, mode="mirror", want_intermediates=True)
    rk, rv = dr.ring()
    slots = np.arange(lo, P) % cfg.ring_capacity
    gk = rk[0, 0].float().cpu().numpy()[:, slots, :]
    gv = rv[0, 0].float().cpu().numpy()[:, :, slots].transpose(0, 2, 1)
    ek = Hn.assert_close(gk, ref["ctx_k"][0], "ring K")
    ev = Hn.assert_close(gv, ref["ctx_v"][0], "ring V")
    g = logits[0].cpu().numpy()
    el = Hn.assert_close(g, ref["logits"], "logits")
    Hn.topk_self_consistent(g, ids[0].cpu().numpy())
    comp, _ = Hn.topk_agrees_away_from_ties(ref["logits"], ids[0].cpu().numpy(), 16, gpu_logits=g)
    print(f"ring K err {ek:.3g}, V err {ev:.3g}, logits err {el:.3g}, top-k ranks compared {comp}", flush=True)
    assert comp > 0


def test_prefill_matches_split_staging_tiny():
    """The same 300 rows staged in one prefill call and in chunks of 100 rows
    (split-K path): ring contents agree to the bf16 tolerance."""
    binding = _gpu()
    W, P = 300, 300
    cfg = config.tiny(window=W, max_stage_rows=600)
    w = synth.make_weights(cfg, seed=8, device="cuda")
    taps = synth.make_taps(cfg, P, seed=9, device="cuda")
    rings = []
    for chunk in (W, 100):
        dr = binding.Drafter(cfg, w)
        dr.reset(0, 0, P)
        for r0 in range(0, W, chunk):
            n = min(chunk, W - r0)
            dr.tap_stage([t[r0:r0 + n] for t in taps], n, req_of_row=torch.zeros(n, dtype=torch.int32, device="cuda"),
                         pos_of_row=torch.arange(r0, r0 + n, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert dr.check() == 0
        rk, rv = dr.ring()
        rings.append((rk[:, 0, :, :P].float().cpu().numpy(), rv[:, 0, :, :, :P].float().cpu().numpy()))
    Hn.assert_close(rings[0][0], rings[1][0], "ring K prefill vs split")
    Hn.assert_close(rings[0][1], rings[1][1], "ring V prefill vs split")
