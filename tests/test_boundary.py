"""The C-ABI library loads, exports every function include/dflash.h declares,
and its host-side guards reject bad configurations before any device work (no
GPU needed: these calls make no HIP calls)."""
import ctypes

import pytest

from block_diffusion_drafter_tap_amd import binding as Bd
from block_diffusion_drafter_tap_amd import config


def test_library_exports_every_header_function():
    lib = Bd.load()
    names = Bd.header_functions()
    assert {"dflash_tap_stage", "dflash_draft_block", "dflash_accept"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def _create(cfg, weights=None):
    lib = Bd.load()
    c = Bd.c_config(cfg)
    w = weights if weights is not None else _fake_weights(cfg)
    ctx = ctypes.c_void_p()
    rc = lib.dflash_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(ctx))
    if rc == 0:
        lib.dflash_destroy(ctx)
    return rc, Bd.last_error()


_keep = []


def _fake_weights(cfg):
    """Non-null fake device pointers: create() only checks presence, it never dereferences."""
    w = Bd.dflash_weights()
    fake = 0x1000
    for n in ("embed", "lm_head", "fc", "ctx_norm", "final_norm"):
        setattr(w, n, fake)
    for n in ("wqkv", "wo", "wgu", "wd", "ln_in", "ln_post", "q_norm", "k_norm"):
        arr = (ctypes.c_void_p * cfg.n_layers)(*([fake] * cfg.n_layers))
        _keep.append(arr)
        setattr(w, n, ctypes.cast(arr, Bd.PP))
    return w


def test_valid_configs_create_and_size():
    for cfg in (config.tiny(), config.qwen3_4b(), config.qwen3_4b_hc()):
        rc, msg = _create(cfg)
        assert rc == 0, msg
        assert Bd.state_bytes(cfg) > 0 and Bd.workspace_bytes(cfg) > 0
        lay = Bd.state_layout(cfg)
        ring = cfg.n_layers * cfg.max_requests * cfg.n_kv_heads * cfg.ring_capacity * cfg.head_dim * 2
        assert lay["ring_v"] - lay["ring_k"] >= ring and lay["total"] - lay["ring_v"] >= ring
        assert lay["total"] == Bd.state_bytes(cfg)


@pytest.mark.parametrize("change,code,needle", [
    (dict(tap_hidden=512), -2, "tap_hidden"),
    (dict(n_kv_heads=3), -2, "multiple of n_kv_heads"),
    (dict(ring_capacity=64), -2, "ring_capacity"),
    (dict(ring_capacity=100), -2, "ring_capacity"),
    (dict(block=0), -2, "block"),
    (dict(block=65), -2, "block"),
    (dict(mask_id=4096), -2, "mask_id"),
    (dict(n_taps=9), -2, "n_taps"),
    (dict(head_dim=96, n_q_heads=4, n_kv_heads=2), -5, "head_dim"),
    (dict(ffn=700), -5, "multiples of 128"),
    (dict(rope_theta=0.0), -2, "rope_theta"),
    (dict(max_stage_rows=0), -2, "max_stage_rows"),
])
def test_config_guards(change, code, needle):
    cfg = config.tiny().replace(**change)
    rc, msg = _create(cfg)
    assert rc == code, (rc, msg)
    assert needle in msg
    assert Bd.state_bytes(cfg) == 0


def test_gqa_rows_per_kv_head_guard():
    cfg = config.tiny(block=40).replace(ring_capacity=128)     # 2 q heads per kv head * 40 = 80 > 64
    rc, msg = _create(cfg)
    assert rc == -5 and "query rows" in msg


def test_missing_weights_rejected_before_any_buffer():
    cfg = config.tiny()
    w = _fake_weights(cfg)
    w.fc = None
    rc, msg = _create(cfg, w)
    assert rc == -1 and "fc" in msg
    w = _fake_weights(cfg)
    arr = (ctypes.c_void_p * cfg.n_layers)(*([None] * cfg.n_layers))
    _keep.append(arr)
    w.wd = ctypes.cast(arr, Bd.PP)
    rc, msg = _create(cfg, w)
    assert rc == -1 and "wd[0]" in msg
    cfgn = cfg.replace(ctx_norm=1)
    w = _fake_weights(cfgn)
    w.ctx_norm = None
    rc, msg = _create(cfgn, w)
    assert rc == -1 and "ctx_norm" in msg


def test_misaligned_weights_rejected():
    """Every kernel reads weights in 16-byte pieces: create() refuses a weight,
    gain or per-layer pointer that is not 16-byte aligned."""
    cfg = config.tiny()
    w = _fake_weights(cfg)
    w.embed = 0x1002
    rc, msg = _create(cfg, w)
    assert rc == -1 and "16-byte aligned" in msg
    w = _fake_weights(cfg)
    arr = (ctypes.c_void_p * cfg.n_layers)(*([0x1000] * (cfg.n_layers - 1) + [0x1008]))
    _keep.append(arr)
    w.k_norm = ctypes.cast(arr, Bd.PP)
    rc, msg = _create(cfg, w)
    assert rc == -1 and f"k_norm[{cfg.n_layers - 1}]" in msg and "aligned" in msg
    w = _fake_weights(cfg)
    w.lm_head = 0x1010   # 16-byte aligned: accepted
    rc, msg = _create(cfg, w)
    assert rc == 0, msg


def test_unbound_handle_refuses_calls():
    lib = Bd.load()
    cfg = config.tiny()
    c = Bd.c_config(cfg)
    w = _fake_weights(cfg)
    ctx = ctypes.c_void_p()
    assert lib.dflash_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(ctx)) == 0
    try:
        assert lib.dflash_reset(ctx, None, 0, 0, 5) == -8
        assert lib.dflash_draft_block(ctx, None, 0x1000, 1, None, 0x1000, None, 1) == -8
    finally:
        lib.dflash_destroy(ctx)
