"""A draft round (draft block -> stage the verify rows -> accept) captured once
into a HIP graph and replayed must equal the same round launched eagerly, on
every replay. Two handles start from the same state; handle A runs the rounds
eagerly, handle B replays the captured round, with eager work and
synchronizations between the replays. Everything is compared bit-exact: top-k
ids and values, accept outputs, next tokens and positions."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_tap_amd import config, synth

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager_tiny():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_tap_amd import binding
    cfg = config.tiny()
    B, V = cfg.block, cfg.vocab
    print(f"case: tiny graph replay B={B} W={cfg.window}", flush=True)
    w = synth.make_weights(cfg, seed=12, device="cuda")
    P = 90
    taps = synth.make_taps(cfg, P, seed=13, device="cuda")
    vt = synth.make_taps(cfg, B, seed=14, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(15)
    verify = torch.randint(0, V, (1, B), generator=g, device="cuda", dtype=torch.int32)

    def make():
        dr = binding.Drafter(cfg, w)
        dr.reset(0, P - cfg.window, P)
        n = cfg.window
        dr.tap_stage([t[P - n:] for t in taps], n, req_of_row=torch.zeros(n, dtype=torch.int32, device="cuda"),
                     pos_of_row=torch.arange(P - n, P, dtype=torch.int32, device="cuda"))
        bufs = {"tokens": synth.block_tokens(cfg, 1, seed=16, device="cuda"),
                "ids": torch.empty((1, B - 1, 16), dtype=torch.int32, device="cuda"),
                "vals": torch.empty((1, B - 1, 16), dtype=torch.float32, device="cuda")}
        bufs["out"] = {"accept_len": torch.empty(1, dtype=torch.int32, device="cuda"),
                       "emitted": torch.empty((1, B), dtype=torch.int32, device="cuda"),
                       "n_emit": torch.empty(1, dtype=torch.int32, device="cuda"),
                       "next_tokens": bufs["tokens"]}
        return dr, bufs

    def round_(dr, b):
        dr.draft_block(b["tokens"], k=16, ids=b["ids"], vals=b["vals"])
        dr.tap_stage(vt, B, rows_per_req=B)
        dr.accept(b["ids"], 16, verify, out=b["out"])

    A, a = make()
    Bh, b = make()
    torch.cuda.synchronize()
    # one eager round on both (the captured handle warms up on a side stream)
    round_(A, a)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        round_(Bh, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_(Bh, b)
    for rep in range(4):
        round_(A, a)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert A.check() == 0 and Bh.check() == 0
        for key in ("ids", "vals"):
            np.testing.assert_array_equal(a[key].cpu().numpy(), b[key].cpu().numpy(), err_msg=f"replay {rep} {key}")
        for key in ("accept_len", "emitted", "n_emit", "next_tokens"):
            np.testing.assert_array_equal(a["out"][key].cpu().numpy(), b["out"][key].cpu().numpy(),
                                          err_msg=f"replay {rep} {key}")
        pa, pb = A.positions(), Bh.positions()
        assert int(pa[0][0]) == int(pb[0][0]), (rep, pa, pb)
        print(f"replay {rep}: accept {int(a['out']['accept_len'][0])}, pos {int(pa[0][0])}", flush=True)
    del graph
