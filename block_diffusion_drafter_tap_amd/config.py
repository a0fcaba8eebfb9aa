"""Drafter configuration (shapes and scalars only; no arithmetic of the method).

Field meanings follow the C struct ``dflash_config`` in ``include/dflash.h``.
The named workloads are the synthetic stand-ins for the drafters the pages run:
a Qwen3-4B-shaped DFlash drafter ("[RFC] DFlash", ExecuTorch PR #20840,
"Summary" and "Test Plan": Qwen3-4B target, block 16) and the 5-layer DFlash2
drafter with tapped target layers ("feat: DFlash2 block-diffusion drafter for
Qwen 3.8", Mference PR #22, "What's here").
"""
from __future__ import annotations

import dataclasses

WFMT_BF16 = 0
WFMT_INT4_G64 = 1


@dataclasses.dataclass
class DFlashConfig:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_taps: int
    hc_streams: int
    tap_hidden: int
    block: int
    window: int
    ring_capacity: int
    max_requests: int
    mask_id: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    ctx_norm: int = 0
    wfmt: int = WFMT_BF16
    max_stage_rows: int = 256

    @property
    def tap_width(self) -> int:
        """Width of the concatenated (hc-reduced) tap row fed to fc."""
        return self.n_taps * self.tap_hidden

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def replace(self, **kw) -> "DFlashConfig":
        return dataclasses.replace(self, **kw)


def ring_for(window: int, block: int, align: int = 64) -> int:
    """Smallest ring capacity that holds a full window plus one block."""
    need = window + block
    return (need + align - 1) // align * align


def tiny(block: int = 8, window: int = 64, max_requests: int = 1, **kw) -> DFlashConfig:
    """1 draft layer, hidden 256, 4/2 heads of 64, FFN 768, vocab 4096, 2 taps."""
    cfg = DFlashConfig(
        n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768,
        vocab=4096, n_taps=2, hc_streams=1, tap_hidden=256, block=block,
        window=window, ring_capacity=ring_for(window, block),
        max_requests=max_requests, mask_id=4095, max_stage_rows=256)
    return cfg.replace(**kw)


def qwen3_4b(block: int = 16, window: int = 4096, max_requests: int = 1,
             max_stage_rows: int = 4096, **kw) -> DFlashConfig:
    """5 draft layers over a Qwen3-4B-shaped target (hidden 2560, 32/8 heads of
    128, FFN 9728, vocab 151936), 5 tapped layers."""
    cfg = DFlashConfig(
        n_layers=5, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728,
        vocab=151936, n_taps=5, hc_streams=1, tap_hidden=2560, block=block,
        window=window, ring_capacity=ring_for(window, block),
        max_requests=max_requests, mask_id=151935, max_stage_rows=max_stage_rows)
    return cfg.replace(**kw)


def qwen3_8b_int4(block: int = 8, window: int = 2048, max_requests: int = 1,
                  max_stage_rows: int = 2048, **kw) -> DFlashConfig:
    """Qwen3-8B-shaped drafter with INT4 (g64, fp16 scales) projections."""
    cfg = DFlashConfig(
        n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
        vocab=151936, n_taps=5, hc_streams=1, tap_hidden=4096, block=block,
        window=window, ring_capacity=ring_for(window, block),
        max_requests=max_requests, mask_id=151935, max_stage_rows=max_stage_rows,
        wfmt=WFMT_INT4_G64)
    return cfg.replace(**kw)


def qwen3_4b_hc(block: int = 8, window: int = 4096, max_requests: int = 8,
                max_stage_rows: int = 4096, **kw) -> DFlashConfig:
    """Qwen3-4B-shaped drafter fed by 4 hyper-connection streams per tap."""
    return qwen3_4b(block=block, window=window, max_requests=max_requests,
                    max_stage_rows=max_stage_rows, hc_streams=4, **kw)
