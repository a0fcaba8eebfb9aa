"""The Python wrappers refuse wrong tensors before any pointer reaches the C ABI
(no GPU): the library cannot check buffer sizes itself, so an undersized or
mistyped tensor would otherwise be read or written out of bounds on the device."""
import pytest
import torch

from block_diffusion_drafter_tap_amd import binding, config


class _NoLib:
    def __getattr__(self, name):
        raise AssertionError(f"the C ABI was reached ({name}) with an invalid argument")


@pytest.fixture
def dr():
    d = object.__new__(binding.Drafter)
    d.cfg = config.tiny(max_requests=2)
    d.device = torch.device("cpu")
    d.lib = _NoLib()
    d.ctx = None
    d._keep = []
    return d


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def test_draft_block_argument_checks(dr):
    B, V = dr.cfg.block, dr.cfg.vocab
    with pytest.raises(ValueError, match="int32"):
        dr.draft_block(torch.zeros((1, B), dtype=torch.int64), k=1)
    with pytest.raises(ValueError, match="shape"):
        dr.draft_block(_i32(1, B + 1), k=1)
    with pytest.raises(ValueError, match="logits"):
        dr.draft_block(_i32(1, B), k=1, logits=_f32(1, B, V))
    with pytest.raises(ValueError, match="ids"):
        dr.draft_block(_i32(1, B), k=16, ids=_i32(1, B - 1, 1))
    with pytest.raises(ValueError, match="vals"):
        dr.draft_block(_i32(1, B), k=16, ids=_i32(1, B - 1, 16), vals=_f32(1, B - 1, 8))
    with pytest.raises(ValueError, match="contiguous"):
        dr.draft_block(_i32(1, 2 * B)[:, ::2], k=1)
    # right shapes, host memory: refused as not on the device
    with pytest.raises(ValueError, match="device"):
        dr.draft_block(_i32(1, B), k=16, ids=_i32(1, B - 1, 16))
    with pytest.raises(ValueError, match="shape"):
        dr.draft_block_n(_i32(1, 3), k=1, logits=_f32(1, 3, V))


def test_accept_argument_checks(dr):
    B = dr.cfg.block
    with pytest.raises(ValueError, match="verify_ids"):
        dr.accept(_i32(1, B - 1, 1), 1, _i32(1, B - 1))
    with pytest.raises(ValueError, match="draft_ids"):
        dr.accept(_i32(1, B - 1, 1), 16, _i32(1, B))
    with pytest.raises(ValueError, match="budget"):
        dr.accept(_i32(1, B - 1, 1), 1, _i32(1, B), budget=_i32(2))
    with pytest.raises(ValueError, match="emitted"):
        dr.accept(_i32(1, B - 1, 1), 1, _i32(1, B),
                  out={"accept_len": _i32(1), "emitted": _i32(1, B - 1), "n_emit": _i32(1)})
    with pytest.raises(ValueError, match="int32"):
        dr.accept_n(_i32(1, 2, 1), 1, torch.zeros((1, 3), dtype=torch.int64))
    with pytest.raises(ValueError, match="device"):
        dr.accept(_i32(1, B - 1, 1), 1, _i32(1, B))


def test_tap_stage_argument_checks(dr):
    c = dr.cfg
    taps = [_f32(10, c.tap_hidden) for _ in range(c.n_taps)]
    with pytest.raises(ValueError, match="expected"):
        dr.tap_stage(taps[:1], 10, rows_per_req=10)
    with pytest.raises(ValueError, match="rows"):
        dr.tap_stage(taps, 11, rows_per_req=11)
    with pytest.raises(ValueError, match="float32"):
        dr.tap_stage([t.double() for t in taps], 10, rows_per_req=10)
    with pytest.raises(ValueError, match=">= 256"):
        dr.tap_stage([t[:, :100] for t in taps], 10, rows_per_req=10)
    with pytest.raises(ValueError, match="pos_of_row"):
        dr.tap_stage(taps, 10, req_of_row=_i32(10), pos_of_row=_i32(9))
    with pytest.raises(ValueError, match="device"):
        dr.tap_stage(taps, 10, rows_per_req=10)


def test_verify_and_advance_argument_checks(dr):
    c = dr.cfg
    with pytest.raises(ValueError, match="block_tokens"):
        dr.verify_block(torch.zeros((1, 4), dtype=torch.int64))
    with pytest.raises(ValueError, match="logits"):
        dr.verify_block(_i32(1, 4), logits=_f32(1, 3, c.vocab))
    with pytest.raises(ValueError, match="same length"):
        dr.verify_block(_i32(1, 4), [0], [])
    with pytest.raises(ValueError, match="rows"):
        dr.verify_block(_i32(1, 4), [0], [_f32(3, c.hidden)])
    with pytest.raises(ValueError, match="int32"):
        dr.advance(torch.zeros(2, dtype=torch.int64))


def test_block_policy_host_functions_match_the_oracle():
    """dflash_policy_init/next/update (host code of the library) against the
    oracle's adaptive block policy over random accept sequences."""
    import numpy as np

    from block_diffusion_drafter_tap_amd import binding as Bd
    from oracle import sampling as S
    rng = np.random.default_rng(0)
    for block in (1, 2, 3, 8, 16):
        for w in (0.5, 0.25, 1.0):
            p, q = Bd.BlockPolicy(block, w), S.BlockPolicy(block, w)
            for _ in range(200):
                b = p.next_block()
                assert b == q.next_block() and 1 <= b <= max(block, 1)
                a = int(rng.integers(0, max(b, 1)))
                p.update(a)
                q.update(a)
                assert p.mean == q.mean


def test_block_policy_stays_in_range_for_any_accept_value():
    from block_diffusion_drafter_tap_amd import binding as Bd
    for acc in (10 ** 9, -10 ** 9, 2 ** 31 - 1, -2 ** 31):
        p = Bd.BlockPolicy(8, 1.0)
        p.update(acc)
        assert 2 <= p.next_block() <= 8
    p = Bd.BlockPolicy(8, float("nan"))
    p.update(3)
    assert p.next_block() == 2


def test_sampled_accept_argument_checks(dr):
    import torch
    V = dr.cfg.vocab
    z = torch.zeros((2, 4, V), dtype=torch.float32)
    with pytest.raises(ValueError, match="target_logits"):
        dr.accept_sampled(torch.zeros((2, 3), dtype=torch.int32), 1, torch.zeros((2, 4), dtype=torch.float32))
    with pytest.raises(ValueError, match="target_logits"):
        dr.accept_sampled(torch.zeros((2, 3), dtype=torch.int32), 1, torch.zeros((2, 4, V - 1), dtype=torch.float32))
    with pytest.raises(ValueError, match="draft_ids"):
        dr.accept_sampled(torch.zeros((2, 2), dtype=torch.int32), 1, z)
    with pytest.raises(ValueError, match="budget"):
        dr.accept_sampled(torch.zeros((2, 3), dtype=torch.int32), 1, z, budget=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="device"):
        dr.accept_sampled(torch.zeros((2, 3), dtype=torch.int32), 1, z)
