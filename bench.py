#!/usr/bin/env python3
"""Throughput of the DFlash draft round on one MI355X.

A step is one round of the hot path for every request: dflash_draft_block
(5 draft layers + LM head + top-16) -> synthetic target verify ids (torch ops
on the device, part of the timed loop) -> dflash_tap_stage of the B verify rows
-> dflash_accept. Inputs are seeded synthetic tensors resident in HBM before
timing starts. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload c3|c2|c3b8|c5]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure (no sparsity)
COPY_BYTES = 512 << 20   # calibration copy read (and written) once before warm-up
# rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the LM-head kernel at the default workload
LM_PROFILE = os.path.join(ROOT, "profiles", "lm_logits_qwen3-4b_b16_ctx4k.md")
LM_SOURCES = [os.path.join(ROOT, "block_diffusion_drafter_tap_amd", "csrc", f)
              for f in ("lmhead.hip", "norm_stage.h", "device.h", "kernels.h")]


def lm_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in LM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def lm_traffic(workload: str):
    """HBM bytes per LM-head launch measured by the committed counter summary,
    or None when that summary is absent, covers another workload, or was taken
    with different LM-head sources than the ones built now."""
    if workload != "c3" or not os.path.exists(LM_PROFILE):
        return None
    fields = {}
    with open(LM_PROFILE) as fh:
        for line in fh:
            text = line.strip().lstrip("-").strip().strip("`")
            if text.startswith(("source_sha256:", "traffic_bytes_per_launch:")):
                key, val = text.split(":", 1)
                fields[key.strip()] = val.split("`")[0].strip()
    if fields.get("source_sha256") != lm_sources_sha256():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


WORKLOADS = {
    # name: (config builder, builder kwargs, requests, k, description)
    "c3": ("qwen3_4b", dict(block=16, window=4096), 1, 16,
           "qwen3-4b-shaped drafter (5 layers, hidden 2560, 32/8 heads x 128, ffn 9728, vocab 151936, 5 taps), "
           "block 16, context window 4096 rows staged from a 16384-row tap buffer, top-16, 1 request"),
    "c3b8": ("qwen3_4b", dict(block=8, window=4096), 1, 16,
             "qwen3-4b-shaped drafter, block 8, context window 4096, top-16, 1 request"),
    "c2": ("qwen3_4b", dict(block=16, window=1024), 1, 1,
           "qwen3-4b-shaped drafter, block 16, context 1024 rows, argmax, 1 request"),
    "c4": ("qwen3_8b_int4", dict(block=8, window=2048), 1, 1,
           "qwen3-8b-shaped drafter with INT4 g64 projections (5 layers, hidden 4096, 32/8 heads x 128, "
           "ffn 12288, bf16 LM head vocab 151936), block 8, context 2048, argmax, 1 request"),
    "c4b6": ("qwen3_8b_int4", dict(block=6, window=2048), 1, 1,
             "qwen3-8b-shaped drafter with INT4 g64 projections, block 6, context 2048, argmax, 1 request"),
    "c5": ("qwen3_4b", dict(block=8, window=4096, max_requests=8, hc_streams=4), 8, 1,
           "qwen3-4b-shaped drafter fed by 4 hyper-connection streams per tap, block 8, "
           "8 requests with their own 4096-row contexts, argmax"),
}


def lm_kernel_label(hidden: int, vocab: int, rows: int) -> str:
    """Name of the LM-head logits kernel the library launches for this shape, as
    its planner picks it on 256 compute units: up to 16 rows, the normed rows
    (8 of them when there are at most 8) staged in LDS in 1 or 2 phases of K
    beside a ring of 16 weight slots (8 waves
    x 2 chunks x 4 KB); 17..64 rows, bf16 normed rows and weights both loaded
    straight into LDS in phases of whole 128-column chunks; otherwise the
    windowed kernel. The 16-row kernel deals out 16-row weight tiles, at most 8
    per wave; the 17..64-row kernel takes at most 5 column groups of 128 per
    workgroup."""
    groups = (vocab + 127) // 128
    per = -(-groups // 256)
    tiles = (vocab + 15) // 16
    nch = hidden // 128 if hidden % 128 == 0 else 0
    if rows <= 16 and nch and tiles <= 8 * min(256, tiles) * 8:
        rx = 8 if rows <= 8 else 16   # rows staged
        for kph in (1, 2):
            kw = hidden // kph
            if hidden % kph or kw % 128 or kw // 128 < 2 or kw // 8 > 10 * (512 // rx):
                continue
            lds = ((rx * (kw + 8) * 2 + 15) & ~15) + ((kw * 2 + 1023) & ~1023) + 8 * 2 * 4096 + 2048
            if lds <= 160 * 1024:
                return "lm_logits_lds_kernel (shared LM head logits + 16-column maxima, weights streamed through LDS)"
    if 16 < rows <= 64 and nch and per <= 5:
        npcs = (2,) if rows > 32 else (5, 4)
        if any(nch % n == 0 for n in npcs):
            return ("lm_logits_dma_kernel (shared LM head logits + 16-column maxima, normed rows and weights "
                    "loaded straight into LDS)")
    return "lm_logits_kernel (shared LM head logits + 16-column maxima)"


def round_bytes(cfg, R: int, k: int) -> dict:
    """Algorithmic HBM bytes of one round: every weight once, each request's
    context K/V window read once per layer, new ring rows written, taps read,
    embeddings gathered, ids written."""
    from block_diffusion_drafter_tap_amd import config

    H, hd, L = cfg.hidden, cfg.head_dim, cfg.n_layers
    # bytes per projection weight: bf16, or a nibble plus an fp16 scale per 64
    wb = 0.5 + 2.0 / 64 if cfg.wfmt == config.WFMT_INT4_G64 else 2
    layer_w = int((cfg.qkv_rows * H + H * cfg.n_q_heads * hd + 2 * cfg.ffn * H + H * cfg.ffn) * wb) \
        + 4 * H * 2 + 2 * hd * 2
    fc = int(H * cfg.tap_width * wb)
    lm = cfg.vocab * H * 2
    keys = cfg.window + cfg.block
    ring_read = R * L * 2 * cfg.n_kv_heads * keys * hd * 2
    ring_write = R * L * 2 * cfg.n_kv_heads * hd * 2 * (2 * cfg.block)
    taps = R * cfg.block * cfg.n_taps * cfg.hc_streams * cfg.tap_hidden * 4
    embed = R * cfg.block * H * 2
    out = R * (cfg.block - 1) * k * 8
    total = L * layer_w + fc + lm + ring_read + ring_write + taps + embed + out
    return {"total": total, "lm_head": lm + R * cfg.block * H * 2 + out, "layers": L * layer_w, "fc": fc,
            "ring_read": ring_read}


def class_bytes(cfg, R: int) -> dict:
    """Algorithmic HBM bytes per launch of each timed kernel class: a projection's
    weights (bf16, or packed INT4 with its scales), attention's context and block
    K/V of every request, fc's weights and tap rows, the layer-batched context K/V
    staging's weights, the LM head's bytes as in round_bytes."""
    from block_diffusion_drafter_tap_amd import config

    H, hd, L = cfg.hidden, cfg.head_dim, cfg.n_layers
    wb = 0.5 + 2.0 / 64 if cfg.wfmt == config.WFMT_INT4_G64 else 2
    keys = cfg.window + cfg.block
    return {"qkv": int(cfg.qkv_rows * H * wb), "attn": R * cfg.n_kv_heads * keys * hd * 2 * 2,
            "o": int(H * cfg.n_q_heads * hd * wb), "gate_up": int(2 * cfg.ffn * H * wb),
            "down": int(H * cfg.ffn * wb),
            "fc": int(H * cfg.tap_width * wb) + R * cfg.block * cfg.n_taps * cfg.hc_streams * cfg.tap_hidden * 4,
            "stage_kv": int(L * 2 * cfg.n_kv_heads * hd * H * wb)}


def verify_report(cfg, dev, n_layers: int = 36, steps: int = 20) -> dict:
    """One causal verify pass of a target with the drafter's layer shape at
    Qwen3-4B depth (36 layers): the block's B rows at context W, every row's
    argmax, the residual rows after 5 evenly spaced layers copied out as the
    drafter's taps. The target's ring is zeroed (the pass reads W context rows
    whatever they hold, so the timing is that of real contents)."""
    import torch
    from block_diffusion_drafter_tap_amd import binding, synth

    B, W, H, hd = cfg.block, cfg.window, cfg.hidden, cfg.head_dim
    tcfg = cfg.replace(n_layers=n_layers, max_requests=1)
    w = synth.make_weights(tcfg, seed=7, device=dev)
    tg = binding.Drafter(tcfg, w, target=True)
    tg.state.zero_()
    tg.reset(0, 0, W)
    T = cfg.n_taps
    tap_layers = [1 + i * (n_layers - 3) // (T - 1) for i in range(T)] if T > 1 else [n_layers - 1]
    taps = [torch.empty((B, H), dtype=torch.float32, device=dev) for _ in tap_layers]
    tokens = synth.block_tokens(tcfg, 1, seed=3, device=dev)
    for _ in range(3):
        tg.verify_block(tokens, tap_layers, taps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        tg.verify_block(tokens, tap_layers, taps)
    e1.record()
    torch.cuda.synchronize()
    word = tg.check()
    if word != 0:
        raise SystemExit(f"device error word 0x{word:x} in the verify pass")
    ms = e0.elapsed_time(e1) / steps
    # the same pass replayed from a HIP graph: its ~430 dependent launches no
    # longer wait on the host, whose launch rate differs between machines
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            tg.verify_block(tokens, tap_layers, taps)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            tg.verify_block(tokens, tap_layers, taps)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
        del g
    except RuntimeError:
        graph_ms = None
    layer_w = (tcfg.qkv_rows * H + H * tcfg.n_q_heads * hd + 3 * tcfg.ffn * H) * 2 + 4 * H * 2 + 2 * hd * 2
    kv = n_layers * 2 * tcfg.n_kv_heads * hd * 2
    nbytes = (n_layers * layer_w + tcfg.vocab * H * 2 + kv * (W + B) + kv * B + len(tap_layers) * B * H * 4
              + B * H * 2 + B * 4)
    gbps = nbytes / (ms / 1e3) / 1e9
    del tg, w
    torch.cuda.empty_cache()
    return {"target": f"{n_layers} layers of the drafter's shape (hidden {H}, {tcfg.n_q_heads}/{tcfg.n_kv_heads} "
                      f"heads x {hd}, ffn {tcfg.ffn}), vocab {tcfg.vocab}, causal",
            "rows": B, "context": W, "tap_layers": tap_layers, "ms": round(ms, 4), "bytes": int(nbytes),
            "achieved_gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "graph_ms": None if graph_ms is None else round(graph_ms, 4),
            "graph_frac": None if graph_ms is None else round(nbytes / (graph_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}


def graph_us(fn, reps: int = 20, inner: int = 10):
    """Microseconds per call of fn replayed from a HIP graph: inner calls
    captured once, the graph replayed reps times between HIP events, so the
    figure is the device time of the calls' launches, without the host's
    per-call work or a graph launch per call. None when capture fails."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(inner):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / (reps * inner) * 1e3
        del g
        return round(us, 2)
    except RuntimeError:
        return None


def tree_report(cfg, dr, tokens, k: int, dev, node_counts=(16, 32, 64), rounds: int = 200, seed: int = 5) -> dict:
    """Candidate trees from this drafter's top-16 lists: the mean tokens per
    round of trees of node_counts verify rows against the top-1 chain (block
    rows) under a synthetic target, and the time of the tree build and tree
    accept kernels (back-to-back launches of the largest tree). The synthetic
    target's token at draft position d is the drafter's rank-j candidate: rank 0
    with probability 0.75 (the chain's geometric accept profile), a listed rank
    1..15 with probability 0.2 (rank j with weight 2^-j), otherwise a token
    outside the list. Every tree and the chain walk the same draws. The tree
    takes the whole top-1 chain first, so with block B a tree gains over the
    chain only beyond B nodes."""
    import numpy as np
    import torch
    from block_diffusion_drafter_tap_amd import binding, config, synth

    B = cfg.block
    if k != 16 or B < 2:
        return None
    ids = torch.empty((1, B - 1, 16), dtype=torch.int32, device=dev)
    vals = torch.empty((1, B - 1, 16), dtype=torch.float32, device=dev)
    blk = tokens[:1].contiguous()
    # an accept-only handle of the same block (the accept needs the block, the mask id and positions)
    acfg = config.tiny(block=B)
    acc_h = binding.Drafter(acfg, synth.make_weights(acfg, seed=0, device=dev), device=dev)
    rng = np.random.default_rng(seed)
    w_rank = 0.5 ** np.arange(1, 16)
    w_rank /= w_rank.sum()
    tau = {n: 0 for n in node_counts}
    tau_chain = 0
    for _ in range(rounds):
        dr.draft_block(blk, k=16, ids=ids, vals=vals)
        u = rng.random(B - 1)
        ranks = np.where(u < 0.75, 0, np.where(u < 0.95, 1 + rng.choice(15, size=B - 1, p=w_rank), -1))
        il = ids[0].cpu().numpy()
        g = np.array([il[d, r] if r >= 0 else cfg.vocab + d for d, r in enumerate(ranks)] + [0], dtype=np.int32)
        tau_chain += 1 + int(next((d for d, r in enumerate(ranks) if r != 0), B - 1))
        for n in node_counts:
            tok, par, dep = dr.tree_build(blk, ids, vals, n)
            verify = torch.from_numpy(g[np.minimum(dep[0].cpu().numpy(), B - 1)]).view(1, -1).to(dev)
            acc_h.reset(0, 0, 100)
            tau[n] += int(acc_h.tree_accept(tok, par, verify)["n_emit"][0])
    n = max(node_counts)
    tok, par, dep = dr.tree_build(blk, ids, vals, n)
    verify = torch.zeros((1, n), dtype=torch.int32, device=dev)
    acc_h.reset(0, 0, 100)
    build_us = graph_us(lambda: dr.tree_build(blk, ids, vals, n))
    accept_us = graph_us(lambda: acc_h.tree_accept(tok, par, verify))
    del acc_h
    return {"rounds": rounds, "block": B, "tau_chain": round(tau_chain / rounds, 3),
            "tau_tree": {str(m): round(tau[m] / rounds, 3) for m in node_counts},
            "target_model": "synthetic: the target's token is the drafter's rank-0 candidate w.p. 0.75, "
                            "a listed rank 1..15 (weight 2^-j) w.p. 0.2, unlisted otherwise",
            "timed_nodes": n, "build_us": build_us, "accept_us": accept_us, "timing": "HIP graph replay"}


def sampling_report(cfg, dev) -> dict:
    """Sampling-mode accept (typical acceptance 0.2, T 1.0, top-p 0.95, top-k
    20) over one block of verify logits [R, B, V] fp32: the device time of its
    three kernels (HIP graph replay) and its rate against the logits' bytes
    (read once algorithmically)."""
    import torch
    from block_diffusion_drafter_tap_amd import binding, config, synth

    R, B, V = cfg.max_requests, cfg.block, cfg.vocab
    acfg = config.tiny(block=B, max_requests=R).replace(vocab=V)
    h = binding.Drafter(acfg, synth.make_weights(acfg, seed=0, device=dev), device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    z = torch.randn((R, B, V), generator=g, device=dev) * 2.0
    d = torch.argmax(z[:, : B - 1], dim=2).to(torch.int32).contiguous()
    us = graph_us(lambda: h.accept_sampled(d, 1, z, temperature=1.0, top_k=20, top_p=0.95, eps=0.2, seed=1,
                                            round=7))
    if us is None:
        return None
    nbytes = R * B * V * 4
    del h
    return {"logits_shape": [R, B, V], "us": round(us, 2), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "params": "typical 0.2, T 1.0, top-p 0.95, top-k 20", "timing": "HIP graph replay"}


def prefill_report(cfg, rows: int, ms: float) -> dict:
    """Prefill staging of one request's window (fc over the gathered taps, then
    every layer's context K/V into the ring): a dense contraction, reported
    against the dense bf16 MFMA peak."""
    H = cfg.hidden
    flops = 2.0 * rows * cfg.tap_width * H + 2.0 * rows * H * 2 * cfg.n_kv_heads * cfg.head_dim * cfg.n_layers
    tfs = flops / (ms / 1e3) / 1e12
    return {"rows": rows, "ms": round(ms, 3), "gflop": round(flops / 1e9, 1), "tflops": round(tfs, 1),
            "bound": "mfma", "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)}


def cpu_baseline(cfg, w, taps_hist, tokens, pos, valid_from, budget_s: float = 15.0) -> dict:
    """The oracle (fp64 NumPy, as it stands) timed on this host for a bounded
    sample: whole draft rounds of request 0 at the benchmark's shapes, repeated
    until `budget_s` of CPU time has passed (at least one)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import dflash as D
    from block_diffusion_drafter_tap_amd import synth

    def host(t):
        return t.cpu().numpy() if t.dtype == torch.uint8 else synth.bf16_to_f32_numpy(t)

    wh = D.dequantize({kk: ([host(t) for t in v] if isinstance(v, list) else host(v)) for kk, v in w.items()})
    n, t0 = 0, time.perf_counter()
    while True:
        D.draft_block(cfg, wh, taps_hist, tokens, pos, valid_from, mode="mirror")
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 8:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    # one more round on a single BLAS thread when a round is short enough
    one = None
    if el / n <= 5.0:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            t1 = time.perf_counter()
            D.draft_block(cfg, wh, taps_hist, tokens, pos, valid_from, mode="mirror")
            one = round(1.0 / (time.perf_counter() - t1), 4)
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": n / el, "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full draft round(s) of one request (uncached context recompute of the "
                      f"{cfg.window}-row window, {cfg.n_layers} layers, LM head + top-k) in {el:.1f} s",
            "value_1_thread": one, "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-verify", action="store_true", help="skip the target verify-pass measurement")
    ap.add_argument("--no-sweep", action="store_true", help="skip the draft-forward block-length sweep")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the draft round shards by request with no exchange between GPUs", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_drafter_tap_amd import binding, config, synth

    builder, kw, R, k, desc = WORKLOADS[args.workload]
    cfg = getattr(config, builder)(max_stage_rows=kw["window"], **kw)
    B, V, W = cfg.block, cfg.vocab, cfg.window
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    w = synth.make_weights(cfg, seed=0, device=dev)
    dr = binding.Drafter(cfg, w, device=dev)

    # prefill: each request stages the trailing W rows of a 16384-row tap buffer;
    # request 0's staging is timed (HIP events on the launch stream) after a warm-up
    # staging of the same rows. A spin kernel of about 2 ms runs before the first
    # event, so the host has enqueued the whole staging by the time the GPU gets
    # to it: the events bracket the device's time, not the host's submission
    # latency from an idle GPU (about 0.23 ms of Python, binding and launches)
    total_rows = 16384
    start = [total_rows + 37 * r for r in range(R)]
    hist = []
    pre_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for r in range(R):
        taps = synth.make_taps(cfg, total_rows, seed=0, device=dev, stream=r, outliers=(cfg.hc_streams == 1))
        hist.append(taps)
        p0 = start[r]
        dr.reset(r, p0 - W, p0)
        rows = torch.arange(p0 - W, p0, dtype=torch.int32, device=dev)
        req = torch.full((W,), r, dtype=torch.int32, device=dev)
        for rep in range(2 if r == 0 else 1):
            if r == 0 and rep == 1:
                torch.cuda.synchronize()
                torch.cuda._sleep(4_000_000)
                pre_ev[0].record()
            dr.tap_stage([t[total_rows - W:] for t in taps], W, req_of_row=req, pos_of_row=rows)
            if r == 0 and rep == 1:
                pre_ev[1].record()
    torch.cuda.synchronize()
    prefill_ms = pre_ev[0].elapsed_time(pre_ev[1])
    # per-round verify rows come from a pool of 4096 pre-generated rows per request
    pool_rows = 4096
    pool = [synth.make_taps(cfg, pool_rows, seed=1, device=dev, stream=100 + r, outliers=(cfg.hc_streams == 1))
            for r in range(R)]
    pool_cat = [torch.stack([pool[r][t] for r in range(R)], 0) for t in range(cfg.n_taps)]  # [R, rows, width]

    n_rounds = args.warmup + args.steps
    acc = synth.geometric_accepts(n_rounds, R, B, p=0.75, seed=0)
    j = torch.arange(B, device=dev).view(1, 1, B)
    keep = (j < torch.from_numpy(acc).to(dev).view(n_rounds, R, 1))          # [rounds, R, B]
    g = torch.Generator(device=dev).manual_seed(2)
    noise1 = torch.randint(0, V - 1, (n_rounds, R, B), generator=g, device=dev, dtype=torch.int32) + 1
    # per-round offsets of the verify ids: 0 where the target agrees with the draft
    # (j < a), else 1 + noise in [1, V-1], so (draft + offset) mod V differs there
    delta = torch.where(keep, torch.zeros_like(noise1), noise1)[:, :, :B - 1].contiguous()
    # with an even vocabulary the same agreement pattern is one launch: draft XOR 1
    # is another id in [0, V) wherever the target disagrees
    flip = (~keep).to(torch.int32)[:, :, :B - 1].contiguous() if V % 2 == 0 else None

    tokens = synth.block_tokens(cfg, R, seed=0, device=dev)
    ids = torch.empty((R, B - 1, k), dtype=torch.int32, device=dev)
    vals = torch.empty((R, B - 1, k), dtype=torch.float32, device=dev)
    # the last verify id (the bonus token after a full accept) is a fixed token
    verify = torch.ones((R, B), dtype=torch.int32, device=dev)
    vview = verify[:, :B - 1]
    out = {"accept_len": torch.empty(R, dtype=torch.int32, device=dev),
           "emitted": torch.empty((R, B), dtype=torch.int32, device=dev),
           "n_emit": torch.empty(R, dtype=torch.int32, device=dev),
           "next_tokens": tokens}
    row_stride = cfg.hc_streams * cfg.tap_hidden

    def one_round(i: int):
        dr.draft_block(tokens, k=k, ids=ids, vals=vals)
        if flip is not None:
            torch.bitwise_xor(ids[:, :, 0], flip[i], out=vview)
        else:
            torch.add(ids[:, :, 0], delta[i], out=vview)
            vview.remainder_(V)
        off = (i * B) % (pool_rows - B)
        if R == 1:
            ptrs = [pool_cat[t][0, off:].data_ptr() for t in range(cfg.n_taps)]
        else:
            # request r's verify rows are rows [r*B, (r+1)*B) of one staging buffer
            for t in range(cfg.n_taps):
                stage_bufs[t].view(R, B, -1).copy_(pool_cat[t][:, off:off + B])
            ptrs = [stage_bufs[t].data_ptr() for t in range(cfg.n_taps)]
        dr.tap_stage(None, R * B, row_stride=row_stride, rows_per_req=B, ptrs=ptrs)
        dr.accept(ids, k, verify, out=out)

    stage_bufs = [torch.empty((R * B, row_stride), dtype=torch.float32, device=dev) for _ in range(cfg.n_taps)]

    # a plain device copy of known size, so HBM byte counters of a profiled run can be
    # scaled: counter(copy) / 2 * COPY_BYTES is what the counters report for that traffic
    calib_src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    del calib_src, calib_dst

    # dominant kernel timing: HIP events around every LM-head launch in the timed region
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    for i in range(args.warmup):
        one_round(i)
    torch.cuda.synchronize()
    for e in ev_b + ev_a:
        e.record()
    torch.cuda.synchronize()
    dr.set_timing_events(binding.K_LMHEAD, ev_b, ev_a)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.warmup, n_rounds):
        one_round(i)
    t_end.record()
    torch.cuda.synchronize()
    dr.set_timing_events(binding.K_LMHEAD, [], [])
    ms = t_start.elapsed_time(t_end)
    word = dr.check()
    if word != 0:
        raise SystemExit(f"device error word 0x{word:x}")
    lm_ms = float(np.mean([b.elapsed_time(a) for b, a in zip(ev_b, ev_a)]))
    st = dr.stats().cpu().numpy()   # accept profile of the warm-up + timed rounds

    # per-round distribution: a second pass of the same rounds with an event
    # between consecutive rounds (kept out of the headline loop above)
    rev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    for j, i in enumerate(range(args.warmup, n_rounds)):
        rev[j].record()
        one_round(i)
    rev[-1].record()
    torch.cuda.synchronize()
    per_round = np.array([rev[j].elapsed_time(rev[j + 1]) for j in range(args.steps)])

    # per kernel class: HIP events around every launch of the class (a projection's
    # GEMM with its finish kernel, attention with its combine) in one more pass of
    # the same rounds
    L = cfg.n_layers
    classes = [("qkv", binding.K_QKV, L), ("attn", binding.K_ATTN, L), ("o", binding.K_O, L),
               ("gate_up", binding.K_GATEUP, L), ("down", binding.K_DOWN, L), ("fc", binding.K_FC, 1),
               ("stage_kv", binding.K_STAGE_KV, 1)]
    cev = {}
    for name, kc, per in classes:
        cev[name] = ([torch.cuda.Event(enable_timing=True) for _ in range(args.steps * per)],
                     [torch.cuda.Event(enable_timing=True) for _ in range(args.steps * per)])
        for e in cev[name][0] + cev[name][1]:
            e.record()
    torch.cuda.synchronize()
    for name, kc, per in classes:
        dr.set_timing_events(kc, *cev[name])
    for i in range(args.warmup, n_rounds):
        one_round(i)
    torch.cuda.synchronize()
    for name, kc, per in classes:
        dr.set_timing_events(kc, [], [])
    cb = class_bytes(cfg, R)
    rb_lm = round_bytes(cfg, R, k)["lm_head"]
    kernels = {}
    for name, kc, per in classes:
        us = float(np.mean([b.elapsed_time(a) for b, a in zip(*cev[name])])) * 1e3
        gbps = cb[name] / (us * 1e-6) / 1e9
        kernels[name] = {"us": round(us, 2), "launches_per_round": per, "bytes_per_launch": cb[name],
                         "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    kernels["lm_head"] = {"us": round(lm_ms * 1e3, 2), "launches_per_round": 1, "bytes_per_launch": rb_lm,
                          "gbps": round(rb_lm / (lm_ms * 1e-3) / 1e9, 1),
                          "frac": round(rb_lm / (lm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    # the same round captured once into a HIP graph and replayed: launch cost
    # vs plain launches (the replays restage the same verify rows)
    graph = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_round(args.warmup)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_round(args.warmup)
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        word = dr.check()
        if word != 0:
            raise SystemExit(f"device error word 0x{word:x} after graph replays")
        graph = {"ms_per_step": round(gms, 4), "value": round(R / (gms / 1e3), 2), "replays": args.steps}
        del g
    except RuntimeError as exc:   # capture unsupported here: report why, keep the plain result
        graph = {"error": str(exc)[:200]}

    # per-call block length: the draft forward alone at shorter blocks of this handle
    draft_ms_by_block = {}
    for b in ([] if args.no_sweep else sorted({B, B // 2, 4, 2}, reverse=True)):
        if 1 < b <= B:
            tk = tokens[:, :b].contiguous()
            idb = torch.empty((R, b - 1, k), dtype=torch.int32, device=dev)
            for _ in range(3):
                dr.draft_block_n(tk, k=k, ids=idb)
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            b0.record()
            for _ in range(20):
                dr.draft_block_n(tk, k=k, ids=idb)
            b1.record()
            torch.cuda.synchronize()
            draft_ms_by_block[str(b)] = round(b0.elapsed_time(b1) / 20, 4)
    if dr.check() != 0:
        raise SystemExit("device error word set by the block-length sweep")

    # HBM read reference: a plain streaming-read kernel of this library over 1 GiB
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    sink = torch.empty(1024, dtype=torch.int32, device=dev)
    binding.stream_read(src, sink)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record()
    for _ in range(10):
        binding.stream_read(src, sink)
    r1.record()
    torch.cuda.synchronize()
    read_gbps = 10 * src.numel() * 4 / (r0.elapsed_time(r1) / 1e3) / 1e9
    del src, sink

    ms_step = ms / args.steps
    blocks_s = R * args.steps / (ms / 1e3)
    rb = round_bytes(cfg, R, k)
    tau = float(st[B + 1] / max(st[0], 1))
    lm_gbps = rb["lm_head"] / (lm_ms / 1e3) / 1e9
    result = {
        "metric": "DFlash draft blocks/sec + achieved HBM GB/s (block 16, ctx 4K, 1 GPU)",
        "value": round(blocks_s, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) fp32 taps"
                + (" with 0.5% x100 outlier columns" if cfg.hc_streams == 1 else ", 4 hyper-connection streams")
                + ", geometric p=0.75 verify accepts)",
        "config": {"workload": desc, "block": B, "window": W, "requests": R, "topk": k,
                   "layers": cfg.n_layers, "hidden": cfg.hidden, "vocab": V, "hc_streams": cfg.hc_streams,
                   "weights": "int4_g64" if cfg.wfmt == config.WFMT_INT4_G64 else "bf16"},
        "achieved_gbps": round(rb["total"] / (ms_step / 1e3) / 1e9, 1),
        "round_bytes": rb["total"],
        "drafted_tokens_per_s": round(blocks_s * (B - 1), 1),
        "accepted_tokens_per_s": round(blocks_s * tau, 1),
        "tau": round(tau, 3),
        "roofline": {"bound": "hbm", "kernel": lm_kernel_label(cfg.hidden, cfg.vocab, R * B),
                     "achieved": round(lm_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(lm_gbps / HBM_PEAK_GBPS, 4), "traffic": lm_traffic(args.workload),
                     "avg_launch_us": round(lm_ms * 1e3, 2), "bytes_per_launch": rb["lm_head"]},
        "cpu_baseline": None,
        "prefill": prefill_report(cfg, W, prefill_ms),
        "kernels": kernels,
        "round_ms": {"p10": round(float(np.percentile(per_round, 10)), 4),
                     "p50": round(float(np.percentile(per_round, 50)), 4),
                     "p90": round(float(np.percentile(per_round, 90)), 4)},
        "graph": graph,
        "hbm_read_reference_gbps": round(read_gbps, 1),
        "draft_ms_by_block": draft_ms_by_block,
        "verify": None,
        "tree": None,
        "sampling": None,
    }
    if R == 1 and not args.no_sweep:
        result["tree"] = tree_report(cfg, dr, tokens, k, dev)
        result["sampling"] = sampling_report(cfg, dev)
    if not args.no_verify and R == 1 and cfg.wfmt == config.WFMT_BF16:
        result["verify"] = verify_report(cfg, dev)
    if not args.no_cpu_baseline:
        import numpy as np  # noqa: F811
        taps_h = [hist[0][t].cpu().numpy() for t in range(cfg.n_taps)]
        tok = [int(tokens[0, 0])] + [cfg.mask_id] * (B - 1)
        result["cpu_baseline"] = cpu_baseline(cfg, w, [np.asarray(t) for t in taps_h], tok, total_rows,
                                              total_rows - W, budget_s=args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
