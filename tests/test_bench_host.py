"""Host logic of bench.py (no GPU): the one-GPU guard, the committed LM-head
counter summary against the sources built now, and the algorithmic byte counts
the roofline figures divide by."""
import os
import subprocess
import sys

import bench
from block_diffusion_drafter_tap_amd import config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_lm_head_counter_summary_matches_the_sources():
    """roofline.traffic comes from the committed FETCH/WRITE summary only while the
    LM-head sources hash to the value recorded there; a stale summary would make
    the field null on every run."""
    t = bench.lm_traffic("c3")
    assert isinstance(t, int)
    lm = bench.round_bytes(config.qwen3_4b(block=16, window=4096), 1, 16)["lm_head"]
    assert lm <= t <= 1.05 * lm   # the measured bytes: the head once, plus the logits hand-off
    assert bench.lm_traffic("c5") is None


def test_algorithmic_bytes_of_the_benchmark_round():
    """Counted from the shapes: qwen3-4b drafter, block 16, window 4096, top-16, one request."""
    cfg = config.qwen3_4b(block=16, window=4096)
    rb = bench.round_bytes(cfg, 1, 16)
    H, V, F, L = 2560, 151936, 9728, 5
    qkv = (32 + 2 * 8) * 128 * H
    layer = (qkv + H * 32 * 128 + 2 * F * H + H * F) * 2 + 4 * H * 2 + 2 * 128 * 2
    assert rb["layers"] == L * layer
    assert rb["fc"] == H * 5 * H * 2
    assert rb["lm_head"] == V * H * 2 + 16 * H * 2 + 15 * 16 * 8 == 777_996_160
    assert rb["ring_read"] == L * 2 * 8 * (4096 + 16) * 128 * 2
    assert rb["total"] == 1_938_579_840


def test_per_class_bytes_of_the_benchmark_round():
    """Per-launch algorithmic bytes of the kernel classes, counted from the shapes
    (qwen3-4b drafter, block 16, window 4096, one request)."""
    cfg = config.qwen3_4b(block=16, window=4096)
    cb = bench.class_bytes(cfg, 1)
    H, F, hd = 2560, 9728, 128
    assert cb["qkv"] == (32 + 16) * hd * H * 2
    assert cb["o"] == H * 32 * hd * 2
    assert cb["gate_up"] == 2 * F * H * 2 and cb["down"] == H * F * 2
    assert cb["attn"] == 8 * (4096 + 16) * hd * 2 * 2
    assert cb["fc"] == H * 5 * H * 2 + 16 * 5 * H * 4
    assert cb["stage_kv"] == 5 * 2 * 8 * hd * H * 2
