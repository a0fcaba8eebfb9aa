"""GPU verify passes of a causal target (dflash_create_target,
dflash_verify_block, dflash_advance) on the tiny 2-layer target:
  - parity with the oracle target in mirror mode: logits, argmax away from
    ties and the tapped residual rows, for prompt chunks of 8, 8 and 5 rows;
  - batch invariance: a block of 8 rows in one pass equals 8 one-row passes,
    bit for bit (ids and taps);
  - the whole loop on the GPU (target verify -> its taps staged into the
    drafter -> drafter accept -> target advance) equals the GPU target's own
    greedy decoding token for token, with the drafter's drafts and with planted
    drafts that are accepted up to a seeded place."""
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


def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    dcfg = config.tiny(window=64)
    tcfg = config.tiny(window=128).replace(n_layers=2)
    wd = synth.make_weights(dcfg, seed=0, device="cuda")
    wt = synth.make_weights(tcfg, seed=11, device="cuda")
    # a peakier target so greedy continuations vary; drafter and target share embedding and head
    emb = (wd["embed"].float() * 30.0).to(torch.bfloat16)
    wt["embed"], wt["lm_head"] = emb, wd["lm_head"]
    wd["embed"] = emb
    return binding, dcfg, tcfg, wd, wt


def _feed(tg, toks, tap_layers, n_rows=None):
    """One verify pass of `toks` (list) on target handle tg: (ids, taps, logits)."""
    b = len(toks)
    H = tg.cfg.hidden
    taps = [torch.empty((b, H), dtype=torch.float32, device="cuda") for _ in tap_layers]
    logits = torch.empty((1, b, tg.cfg.vocab), dtype=torch.float32, device="cuda")
    ids = tg.verify_block(torch.tensor([toks], dtype=torch.int32, device="cuda"), tap_layers, taps, logits)
    return ids, taps, logits


def test_verify_vs_oracle_target_tiny():
    binding, dcfg, tcfg, wd, wt = _setup()
    print("case: tiny target verify vs mirror oracle target", flush=True)
    tg = binding.Drafter(tcfg, wt, target=True)
    tg.reset(0, 0, 0)
    ref = T.TinyTarget(tcfg, _np(wt), n_layers=2, mode="mirror")
    prompt = [5, 17, 300, 4000, 12, 99, 7, 8, 1, 2, 3, 4, 55, 66, 77, 88, 9, 10, 11, 12, 13]
    pos = 0
    for n in (8, 8, 5):
        chunk = prompt[pos:pos + n]
        ids, taps, logits = _feed(tg, chunk, [0, 1])
        torch.cuda.synchronize()
        assert tg.check() == 0
        ids_o, taps_o, lg_o = ref.feed(chunk, pos, want_logits=True)
        g = logits[0].cpu().numpy()
        el = Hn.assert_close(g, lg_o, f"logits rows {pos}..")
        comp, excl = Hn.topk_agrees_away_from_ties(lg_o, ids.cpu().numpy().reshape(-1, 1), 1, gpu_logits=g)
        for l in range(2):
            Hn.assert_close(taps[l].cpu().numpy(), taps_o[l], f"tap layer {l} rows {pos}..")
        print(f"rows {pos}..{pos + n - 1}: logits err {el:.3g}, argmax compared {comp}, near-ties {excl}", flush=True)
        tg.advance(torch.tensor([n], dtype=torch.int32, device="cuda"))
        pos += n
    assert int(tg.positions()[0][0]) == pos


def test_verify_batch_invariance_tiny():
    binding, dcfg, tcfg, wd, wt = _setup()
    print("case: tiny target, one 8-row pass vs 8 one-row passes", flush=True)
    prompt = [5, 17, 300, 4000, 12, 99, 7, 8, 1, 2]
    nxt = [44, 45, 46, 47, 48, 49, 50, 51]
    out = []
    for mode in ("block", "rows"):
        tg = binding.Drafter(tcfg, wt, target=True)
        tg.reset(0, 0, 0)
        _feed(tg, prompt[:8], [0, 1])
        tg.advance(torch.tensor([8], dtype=torch.int32, device="cuda"))
        _feed(tg, prompt[8:], [0, 1])
        tg.advance(torch.tensor([2], dtype=torch.int32, device="cuda"))
        if mode == "block":
            ids, taps, _ = _feed(tg, nxt, [0, 1])
            out.append((ids.cpu().numpy().reshape(-1), [t.cpu().numpy() for t in taps]))
        else:
            ids_all, taps_all = [], [[], []]
            for t in nxt:
                ids, taps, _ = _feed(tg, [t], [0, 1])
                tg.advance(torch.tensor([1], dtype=torch.int32, device="cuda"))
                ids_all.append(int(ids[0, 0]))
                for l in range(2):
                    taps_all[l].append(taps[l].cpu().numpy()[0])
            out.append((np.array(ids_all), [np.stack(t) for t in taps_all]))
        torch.cuda.synchronize()
        assert tg.check() == 0
    np.testing.assert_array_equal(out[0][0], out[1][0])
    for l in range(2):
        np.testing.assert_array_equal(out[0][1][l], out[1][1][l])


@pytest.mark.parametrize("drafts", ["drafter", "planted"])
def test_full_gpu_loop_lossless_tiny(drafts):
    """drafts="drafter": the GPU drafter's top-1 (random weights: mostly
    rejected). drafts="planted": the target's own continuation with one wrong
    token at a seeded place per round (or none), so rounds accept 0..B-1 drafts
    plus the target's token and the target rolls back the rest of its block."""
    binding, dcfg, tcfg, wd, wt = _setup()
    print(f"case: GPU {drafts} drafts + GPU target loop vs GPU target greedy", flush=True)
    prompt = [5, 17, 300, 4000, 12, 99, 7, 8, 1, 2, 3]
    n_new = 36
    B = dcfg.block
    V = dcfg.vocab
    rng = np.random.default_rng(21)

    def prefill(tg, dr):
        pos = 0
        last_ids = None
        while pos < len(prompt):
            chunk = prompt[pos:pos + B]
            ids, taps, _ = _feed(tg, chunk, [0, 1])
            tg.advance(torch.tensor([len(chunk)], dtype=torch.int32, device="cuda"))
            if dr is not None:
                rows = torch.arange(pos, pos + len(chunk), dtype=torch.int32, device="cuda")
                dr.tap_stage(taps, len(chunk), req_of_row=torch.zeros_like(rows), pos_of_row=rows)
            pos += len(chunk)
            last_ids = ids
        return [int(last_ids[0, -1])], pos

    # reference: the GPU target's greedy decoding, one row per pass
    tg = binding.Drafter(tcfg, wt, target=True)
    tg.reset(0, 0, 0)
    ref, pos = prefill(tg, None)
    while len(ref) < n_new + B:
        ids, _, _ = _feed(tg, [ref[-1]], [0, 1])
        tg.advance(torch.tensor([1], dtype=torch.int32, device="cuda"))
        ref.append(int(ids[0, 0]))

    # speculative loop, all on the GPU
    tg = binding.Drafter(tcfg, wt, target=True)
    dr = binding.Drafter(dcfg, wd)
    tg.reset(0, 0, 0)
    dr.reset(0, 0, len(prompt))
    out, pos = prefill(tg, dr)
    rounds = 0
    accepts = []
    while len(out) < n_new:
        blk = D.next_block(out, B, dcfg.mask_id)
        d_ids = dr.draft_block(torch.tensor([blk], dtype=torch.int32, device="cuda"), k=1)
        if drafts == "planted":
            plant = list(ref[len(out):len(out) + B - 1])
            j = int(rng.integers(0, B))            # j == B - 1: every draft right
            if j < B - 1:
                plant[j] = (plant[j] + 1) % V
            d_ids = torch.tensor(plant, dtype=torch.int32, device="cuda").view(1, B - 1, 1)
            accepts.append(j)
        vtok = torch.cat([torch.tensor([blk[0]], dtype=torch.int32, device="cuda"), d_ids[0, :, 0]]).view(1, B)
        H = tcfg.hidden
        taps = [torch.empty((B, H), dtype=torch.float32, device="cuda") for _ in range(2)]
        v_ids = tg.verify_block(vtok, [0, 1], taps)
        dr.tap_stage(taps, B, rows_per_req=B)
        budget = torch.tensor([n_new - len(out)], dtype=torch.int32, device="cuda")
        res = dr.accept(d_ids, 1, v_ids, budget=budget)
        tg.advance(res["n_emit"])
        n = int(res["n_emit"][0])
        out.extend(res["emitted"][0, :n].cpu().tolist())
        pos += n
        rounds += 1
        assert int(dr.positions()[0][0]) == pos and int(tg.positions()[0][0]) == pos
    torch.cuda.synchronize()
    assert dr.check() == 0 and tg.check() == 0
    assert out == ref[:n_new], (out, ref[:n_new])
    if drafts == "planted":
        assert max(accepts) >= 3
    print(f"lossless over {rounds} rounds, {len(out)} tokens", flush=True)


def test_verify_fullsize_vs_oracle_target():
    """Verify pass at the qwen3-4b layer shape (hidden 2560, 32/8 heads x 128, ffn
    9728, vocab 151936; 4 layers, window 4096): a 300-row prompt fed in 16-row
    passes puts the 16-row block in the second 256-key chunk; its logits,
    argmaxes (away from ties) and the taps after layers 1 and 3 are compared with
    the mirror oracle target, which takes the prompt through its batched prefix
    routine."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    tcfg = config.qwen3_4b(block=16, window=4096, max_stage_rows=16).replace(n_layers=4)
    B, V, H = tcfg.block, tcfg.vocab, tcfg.hidden
    print("case: qwen3-4b-shaped 4-layer target, prompt 300, verify block 16", flush=True)
    wt = synth.make_weights(tcfg, seed=21, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(22)
    P = 300
    toks = torch.randint(0, V - 1, (P + B,), generator=g, device="cuda", dtype=torch.int32)
    prompt, blk = toks[:P].cpu().tolist(), toks[P:].cpu().tolist()
    tg = binding.Drafter(tcfg, wt, target=True)
    tg.reset(0, 0, 0)
    for r0 in range(0, P, B):
        n = min(B, P - r0)
        _feed(tg, prompt[r0:r0 + n], [])
        tg.advance(torch.tensor([n], dtype=torch.int32, device="cuda"))
    ids, taps, logits = _feed(tg, blk, [1, 3])
    torch.cuda.synchronize()
    assert tg.check() == 0
    assert int(tg.positions()[0][0]) == P
    ref = T.TinyTarget(tcfg, _np(wt), n_layers=4, mode="mirror")
    ref.prefill(prompt)
    ids_o, taps_o, lg_o = ref.feed(blk, P, want_logits=True)
    gl = logits[0].cpu().numpy()
    el = Hn.assert_close(gl, lg_o, "verify logits")
    comp, excl = Hn.topk_agrees_away_from_ties(lg_o, ids.cpu().numpy().reshape(-1, 1), 1, gpu_logits=gl)
    Hn.topk_self_consistent(gl, ids.cpu().numpy().reshape(-1, 1))
    et = [Hn.assert_close(taps[i].cpu().numpy(), taps_o[l], f"tap after layer {l}") for i, l in enumerate((1, 3))]
    print(f"logits err {el:.3g}, tap errs {et[0]:.3g} {et[1]:.3g}, argmax compared {comp}, near-ties {excl}",
          flush=True)
    assert comp >= 4


def test_verify_multi_request_invariance_tiny():
    """Three requests in one target handle, each from its own start position
    (valid_from = pos = 5r) with its own tokens, advancing by different amounts:
    every verify pass of the 3-request call equals the same pass of a
    single-request handle bit for bit (ids, taps, logits)."""
    binding, dcfg, tcfg, wd, wt = _setup()
    R, b = 3, 8
    tcfg3 = tcfg.replace(max_requests=R)
    print("case: tiny target, 3 requests in one call vs single-request handles", flush=True)
    g = torch.Generator(device="cuda").manual_seed(31)
    V, H = tcfg.vocab, tcfg.hidden
    n_pass = 5
    toks = torch.randint(0, V - 1, (n_pass, R, b), generator=g, device="cuda", dtype=torch.int32)
    adv = torch.tensor([[8, 8, 8], [8, 8, 8], [3, 8, 1], [5, 2, 8], [1, 1, 1]], dtype=torch.int32, device="cuda")

    def run(handle, reqs):
        handle_out = []
        for p in range(n_pass):
            n = len(reqs)
            taps = [torch.empty((n * b, H), dtype=torch.float32, device="cuda") for _ in range(2)]
            logits = torch.empty((n, b, V), dtype=torch.float32, device="cuda")
            ids = handle.verify_block(toks[p, reqs].contiguous(), [0, 1], taps, logits)
            handle.advance(adv[p, reqs].contiguous())
            handle_out.append((ids.cpu().numpy(), [t.cpu().numpy().reshape(n, b, H) for t in taps],
                               logits.cpu().numpy()))
        torch.cuda.synchronize()
        assert handle.check() == 0
        return handle_out

    multi = binding.Drafter(tcfg3, wt, target=True)
    for r in range(R):
        multi.reset(r, 5 * r, 5 * r)
    out_m = run(multi, list(range(R)))
    pos_m = multi.positions()[0].cpu().numpy()
    for r in range(R):
        single = binding.Drafter(tcfg, wt, target=True)
        single.reset(0, 5 * r, 5 * r)
        out_s = run(single, [r])
        assert int(single.positions()[0][0]) == int(pos_m[r]) == 5 * r + int(adv[:, r].sum())
        for p in range(n_pass):
            np.testing.assert_array_equal(out_m[p][0][r], out_s[p][0][0], err_msg=f"ids pass {p} req {r}")
            for l in range(2):
                np.testing.assert_array_equal(out_m[p][1][l][r], out_s[p][1][l][0], err_msg=f"taps pass {p} req {r}")
            np.testing.assert_array_equal(out_m[p][2][r], out_s[p][2][0], err_msg=f"logits pass {p} req {r}")
