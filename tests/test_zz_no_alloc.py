"""The allocation-free draft entry point (dflash_draft_block_noalloc) against
dflash_draft_block on the same handle and inputs: the same kernels with a
static device scratch in place of the bound workspace, so ids, values and
logits must agree bit for bit. Two calls in a row, the second with fewer
requests (a smaller input over the scratch the first call left behind), on the
tiny drafter and on the qwen3-4b shape with the benchmark's top-16 call."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth

pytestmark = pytest.mark.gpu


def _binding():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    return binding


def _stage_contexts(dr, cfg, R, P, seed):
    for r in range(R):
        taps = synth.make_taps(cfg, P, seed=seed, device="cuda", stream=r)
        lo = max(0, P - cfg.window)
        rows = torch.arange(lo, P, dtype=torch.int32, device="cuda")
        dr.reset(r, lo, P + 3 * r)
        dr.tap_stage([t[lo:] for t in taps], P - lo, req_of_row=torch.full_like(rows, r), pos_of_row=rows + 3 * r)


def _compare(dr, tokens, k, with_logits, what):
    R, B = tokens.shape
    V = dr.cfg.vocab
    outs = []
    for fn in (dr.draft_block, dr.draft_block_noalloc):
        ids = torch.full((R, B - 1, k), -7, dtype=torch.int32, device="cuda")
        vals = torch.full((R, B - 1, k), float("nan"), dtype=torch.float32, device="cuda")
        lg = torch.full((R, B - 1, V), float("nan"), dtype=torch.float32, device="cuda") if with_logits else None
        fn(tokens, k=k, logits=lg, ids=ids, vals=vals)
        torch.cuda.synchronize()
        outs.append((ids.cpu().numpy(), vals.cpu().numpy(), None if lg is None else lg.cpu().numpy()))
    assert dr.check() == 0
    (i0, v0, l0), (i1, v1, l1) = outs
    np.testing.assert_array_equal(i1, i0, err_msg=f"{what}: ids")
    np.testing.assert_array_equal(v1, v0, err_msg=f"{what}: values")
    if with_logits:
        np.testing.assert_array_equal(l1, l0, err_msg=f"{what}: logits")
    print(f"{what}: {R} request(s), top-{k}: bit-exact", flush=True)


def test_noalloc_draft_matches_workspace_draft_tiny():
    binding = _binding()
    cfg = config.tiny(max_requests=2)
    print(f"case: tiny, scratch {binding.draft_scratch_bytes(cfg)} bytes", flush=True)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    dr = binding.Drafter(cfg, w)
    _stage_contexts(dr, cfg, 2, 90, seed=31)
    tokens = synth.block_tokens(cfg, 2, seed=32, device="cuda")
    _compare(dr, tokens, 16, True, "tiny call 1")
    _compare(dr, tokens[:1].contiguous(), 1, True, "tiny call 2 (smaller)")


def test_noalloc_draft_matches_workspace_draft_qwen3_4b():
    binding = _binding()
    cfg = config.qwen3_4b(block=16, window=1024, max_requests=2, max_stage_rows=1024)
    need = binding.draft_scratch_bytes(cfg)
    print(f"case: qwen3-4b shape, block 16, window 1024, 2 requests; scratch {need / 2**20:.1f} MiB", flush=True)
    assert 0 < need <= (64 << 20)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    dr = binding.Drafter(cfg, w)
    _stage_contexts(dr, cfg, 2, 1500, seed=33)
    tokens = synth.block_tokens(cfg, 2, seed=34, device="cuda")
    _compare(dr, tokens, 16, False, "qwen3-4b call 1 (ids + values, no logits)")
    _compare(dr, tokens[1:].contiguous(), 16, True, "qwen3-4b call 2 (smaller, with logits)")


def test_noalloc_refuses_configs_beyond_the_static_scratch():
    binding = _binding()
    cfg = config.qwen3_4b(block=8, window=4096, max_requests=8, hc_streams=4, max_stage_rows=8).replace(n_layers=1)
    assert binding.draft_scratch_bytes(cfg) > (64 << 20)
    w = synth.make_weights(cfg, seed=0, device="cuda")
    dr = binding.Drafter(cfg, w)
    tokens = synth.block_tokens(cfg, 1, seed=35, device="cuda")
    with pytest.raises(binding.DFlashError) as ei:
        dr.draft_block_noalloc(tokens, k=1)
    assert ei.value.code == -4
    print(f"refused: {ei.value}", flush=True)
    torch.cuda.synchronize()
    assert dr.check() == 0
