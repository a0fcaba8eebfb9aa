"""Per-call block length on the GPU (dflash_draft_block_n / dflash_accept_n):
a generation whose rounds shrink at the end of the token budget or of the
sequence capacity, with a target-only step and a short block forced early, must
equal the tiny target's greedy decoding; every round's accept must equal the
oracle's, and every shrunk round's drafts must match the oracle drafter's top-1
away from ties."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth
from oracle import dflash as D
from oracle import target as T
from tests import harness as Hn

pytestmark = pytest.mark.gpu


def _np(w):
    return {k: ([synth.bf16_to_f32_numpy(t) for t in v] if isinstance(v, list) else synth.bf16_to_f32_numpy(v))
            for k, v in w.items()}


@pytest.mark.parametrize("max_seq_extra", [None, 19])
def test_dynamic_block_len_loop(max_seq_extra):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    cfg = config.tiny(window=64)
    print(f"case: dynamic block length, max_seq_extra={max_seq_extra}", flush=True)
    wd = synth.make_weights(cfg, seed=0, device="cuda")
    tcfg = cfg.replace(n_layers=2)
    Wt = _np(synth.make_weights(tcfg, seed=11))
    Wd = _np(wd)
    Wt["embed"] = Wd["embed"] * 30.0
    Wt["lm_head"] = Wd["lm_head"]
    wd["embed"] = torch.from_numpy(Wt["embed"]).to(torch.bfloat16).cuda()
    Wd["embed"] = Wt["embed"]
    tgt = T.TinyTarget(tcfg, Wt, n_layers=2)
    prompt = [5, 17, 300, 4000, 12, 99, 7]
    n_new = 29
    max_seq = len(prompt) + (max_seq_extra if max_seq_extra is not None else 10 ** 6)
    n_expect = min(n_new, max_seq - len(prompt) + 1)
    ref = T.greedy(tgt, prompt, n_expect)

    dr = binding.Drafter(cfg, wd)
    tgt.reset()
    ids, taps = tgt.feed(prompt, 0)
    committed = [t.copy() for t in taps]
    pos = len(prompt)
    dr.reset(0, 0, pos)
    rows = torch.arange(0, pos, dtype=torch.int32, device="cuda")
    dr.tap_stage([torch.from_numpy(t).cuda() for t in taps], pos, req_of_row=torch.zeros_like(rows), pos_of_row=rows)
    out = [ids[-1]]
    blocks = []
    while len(out) < n_new:
        b = D.block_len(cfg.block, n_new, len(out), max_seq, pos)
        if len(blocks) == 1:
            b = min(b, 1)     # a target-only step
        elif len(blocks) == 2:
            b = min(b, 3)     # a short block early
        if b < 1:
            break
        blk = D.next_block(out, b, cfg.mask_id)
        tokens = torch.tensor([blk], dtype=torch.int32, device="cuda")
        draft, g_ids = [], None
        if b > 1:
            logits = torch.empty((1, b - 1, cfg.vocab), dtype=torch.float32, device="cuda")
            g_ids = dr.draft_block_n(tokens, k=1, logits=logits)
            draft = g_ids[0, :, 0].cpu().tolist()
            ref_lg = D.draft_block(cfg, Wd, committed, blk, pos, 0, mode="mirror")["logits"]
            Hn.assert_close(logits[0].cpu().numpy(), ref_lg, f"block {b} logits")
            Hn.topk_agrees_away_from_ties(ref_lg, g_ids[0].cpu().numpy(), 1, gpu_logits=logits[0].cpu().numpy())
        verify, vtaps = tgt.feed([blk[0]] + draft, pos)
        vrows = torch.arange(pos, pos + b, dtype=torch.int32, device="cuda")
        dr.tap_stage([torch.from_numpy(t).cuda() for t in vtaps], b, req_of_row=torch.zeros_like(vrows),
                     pos_of_row=vrows)
        budget = torch.tensor([n_new - len(out)], dtype=torch.int32, device="cuda")
        res = dr.accept_n(g_ids, 1, torch.tensor([verify], dtype=torch.int32, device="cuda"), budget=budget)
        ref_acc = D.accept(draft, verify, budget=n_new - len(out))
        n = int(res["n_emit"][0])
        assert n == ref_acc["n_emit"] and int(res["accept_len"][0]) == ref_acc["acc"], (b, n, ref_acc)
        emitted = res["emitted"][0, :n].cpu().tolist()
        assert emitted == ref_acc["emitted"]
        assert res["next_tokens"][0].cpu().tolist() == D.next_block(out + emitted, b, cfg.mask_id)
        tgt.truncate(pos + n)
        committed = [np.concatenate([c, vt[:n]], 0) for c, vt in zip(committed, vtaps)]
        pos += n
        out.extend(emitted)
        blocks.append(b)
        assert int(dr.positions()[0][0]) == pos
        assert pos <= max_seq
    assert dr.check() == 0
    assert out == ref, (out, ref)
    assert blocks[1] == 1 and blocks[-1] < cfg.block
    print(f"blocks per round {blocks}, {len(out)} tokens", flush=True)
