"""ctypes binding of libdflash.so (entry points of include/dflash.h).

Argument marshalling only: tensors are passed as device pointers
(``data_ptr()``) and the current PyTorch stream as the HIP stream; every step of
the round runs in the library's kernels. There is no fallback: if the library
is missing or was built for nothing this device can run, calls fail loudly.

``Drafter`` is a small convenience wrapper owning the state and workspace
tensors of one handle.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, List, Optional, Sequence

import torch

from .config import DFlashConfig

HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB selects another build of the same library (the host-sanitized copy
# in the CPU sanitizer test); there is no fallback when it is missing.
LIB_PATH = os.environ.get("DFLASH_LIB", os.path.join(HERE, "libdflash.so"))
HEADER = os.path.join(os.path.dirname(HERE), "include", "dflash.h")

c_int, c_void_p, c_size_t, c_float, c_ll, c_uint = (ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                                     ctypes.c_float, ctypes.c_longlong, ctypes.c_uint)

STATUS = {0: "DFLASH_OK", -1: "DFLASH_E_ARG", -2: "DFLASH_E_CONFIG", -3: "DFLASH_E_SHAPE",
          -4: "DFLASH_E_CAPACITY", -5: "DFLASH_E_UNSUPPORTED", -6: "DFLASH_E_HIP",
          -7: "DFLASH_E_DEVICE", -8: "DFLASH_E_STATE"}

K_LMHEAD, K_QKV, K_O, K_GATEUP, K_DOWN, K_ATTN, K_FC, K_STAGE_KV = range(8)


class dflash_config(ctypes.Structure):
    _fields_ = [(n, c_int) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn",
                                      "vocab", "n_taps", "hc_streams", "tap_hidden", "block", "window",
                                      "ring_capacity", "max_requests", "mask_id")] + \
               [("rope_theta", c_float), ("rms_eps", c_float), ("ctx_norm", c_int), ("wfmt", c_int),
                ("max_stage_rows", c_int)]


PP = ctypes.POINTER(c_void_p)


class dflash_weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("fc", c_void_p), ("fc_scales", c_void_p),
                ("ctx_norm", c_void_p), ("final_norm", c_void_p),
                ("wqkv", PP), ("wqkv_scales", PP), ("wo", PP), ("wo_scales", PP),
                ("wgu", PP), ("wgu_scales", PP), ("wd", PP), ("wd_scales", PP),
                ("ln_in", PP), ("ln_post", PP), ("q_norm", PP), ("k_norm", PP)]


class dflash_state_layout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("pos", "valid_from", "error", "stats", "ring_k", "ring_v", "total")]


class dflash_sampling(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("top_k", c_int), ("top_p", c_float), ("typical_eps", c_float),
                ("typical_delta", c_float)]


class dflash_block_policy(ctypes.Structure):
    _fields_ = [("block", c_int), ("weight", ctypes.c_double), ("mean", ctypes.c_double)]


class DFlashError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_diffusion_drafter_tap_amd.build`"
                           " (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P = c_void_p
    sig = {
        "dflash_create": (c_int, [ctypes.POINTER(dflash_config), ctypes.POINTER(dflash_weights), ctypes.POINTER(P)]),
        "dflash_destroy": (None, [P]),
        "dflash_state_bytes": (c_size_t, [ctypes.POINTER(dflash_config)]),
        "dflash_workspace_bytes": (c_size_t, [ctypes.POINTER(dflash_config)]),
        "dflash_get_state_layout": (c_int, [ctypes.POINTER(dflash_config), ctypes.POINTER(dflash_state_layout)]),
        "dflash_bind": (c_int, [P, P, P, P]),
        "dflash_reset": (c_int, [P, P, c_int, c_int, c_int]),
        "dflash_tap_stage": (c_int, [P, P, PP, c_ll, c_int, P, P, c_int]),
        "dflash_draft_block": (c_int, [P, P, P, c_int, P, P, P, c_int]),
        "dflash_draft_block_n": (c_int, [P, P, P, c_int, c_int, P, P, P, c_int]),
        "dflash_draft_block_noalloc": (c_int, [P, P, P, c_int, P, P, P, c_int]),
        "dflash_draft_scratch_bytes": (c_size_t, [ctypes.POINTER(dflash_config)]),
        "dflash_accept": (c_int, [P, P, P, c_int, P, c_int, c_int, P, P, P, P, P]),
        "dflash_accept_n": (c_int, [P, P, P, c_int, P, c_int, c_int, c_int, P, P, P, P, P]),
        "dflash_check": (c_int, [P, P, ctypes.POINTER(c_uint)]),
        "dflash_clear_error": (c_int, [P, P]),
        "dflash_set_timing_events": (c_int, [P, c_int, PP, PP, c_int]),
        "dflash_stream_read": (c_int, [P, c_size_t, P, P]),
        "dflash_create_target": (c_int, [ctypes.POINTER(dflash_config), ctypes.POINTER(dflash_weights),
                                         ctypes.POINTER(P)]),
        "dflash_verify_block": (c_int, [P, P, P, c_int, c_int, P, c_int, PP, c_ll, P, P]),
        "dflash_advance": (c_int, [P, P, P, c_int]),
        "dflash_accept_sampled": (c_int, [P, P, P, c_int, P, c_int, c_int, ctypes.POINTER(dflash_sampling),
                                          ctypes.c_ulonglong, c_uint, c_int, P, P, P, P, P]),
        "dflash_policy_init": (None, [ctypes.POINTER(dflash_block_policy), c_int, ctypes.c_double]),
        "dflash_policy_next": (c_int, [ctypes.POINTER(dflash_block_policy)]),
        "dflash_policy_update": (None, [ctypes.POINTER(dflash_block_policy), c_int]),
        "dflash_tree_build": (c_int, [P, P, P, P, P, c_int, c_int, c_int, P, P, P]),
        "dflash_verify_tree": (c_int, [P, P, P, P, P, c_int, c_int, P, c_int, PP, c_ll, P, P]),
        "dflash_tree_accept": (c_int, [P, P, P, P, c_int, P, c_int, c_int, P, P, P, P, P, P, P, P]),
        "dflash_tree_commit": (c_int, [P, P, P, c_int, P, c_int]),
        "dflash_tap_stage_rows": (c_int, [P, P, PP, c_ll, c_int, P, P, P, c_int]),
        "dflash_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def header_functions(path: str = HEADER) -> List[str]:
    """Names of the functions include/dflash.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", text)))


def stream_read(src: torch.Tensor, sink: torch.Tensor):
    """One streaming read of `src` (the HBM read reference), on the current stream."""
    lib = load()
    _check("dflash_stream_read", lib.dflash_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                                        sink.data_ptr(), _stream()))


def last_error() -> str:
    return load().dflash_last_error().decode()


def _check(fn: str, rc: int):
    if rc != 0:
        raise DFlashError(fn, rc, last_error())


def c_config(cfg: DFlashConfig) -> dflash_config:
    c = dflash_config()
    for name, _ in dflash_config._fields_:
        setattr(c, name, getattr(cfg, name))
    return c


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name: str, dtype, shape=None, min_rows=None, optional: bool = False):
    """Checks a tensor argument before any pointer of it reaches the library, which
    cannot check sizes itself: dtype, exact shape (or at least ``min_rows`` rows)
    and a dense layout. Raises ValueError. ``_on_device`` checks the device after
    every argument's shape has been checked."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if min_rows is not None and (t.dim() < 1 or t.shape[0] < min_rows):
        raise ValueError(f"{name} must have at least {min_rows} rows (got {tuple(t.shape)})")
    if shape is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    for name, t in tensors.items():
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise ValueError(f"{name} must be a device (cuda) tensor")
        if isinstance(t, (list, tuple)):
            for i, u in enumerate(t):
                if isinstance(u, torch.Tensor) and not u.is_cuda:
                    raise ValueError(f"{name}[{i}] must be a device (cuda) tensor")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def state_bytes(cfg: DFlashConfig) -> int:
    return load().dflash_state_bytes(ctypes.byref(c_config(cfg)))


def workspace_bytes(cfg: DFlashConfig) -> int:
    return load().dflash_workspace_bytes(ctypes.byref(c_config(cfg)))


def draft_scratch_bytes(cfg: DFlashConfig) -> int:
    return load().dflash_draft_scratch_bytes(ctypes.byref(c_config(cfg)))


def state_layout(cfg: DFlashConfig) -> Dict[str, int]:
    lay = dflash_state_layout()
    _check("dflash_get_state_layout", load().dflash_get_state_layout(ctypes.byref(c_config(cfg)), ctypes.byref(lay)))
    return {n: getattr(lay, n) for n, _ in dflash_state_layout._fields_}


class Drafter:
    """One library handle with its own state and workspace (torch tensors on ``device``)."""

    def __init__(self, cfg: DFlashConfig, weights: Dict[str, object], device="cuda", target: bool = False):
        self.lib = load()
        self.target = target
        self.cfg = cfg
        self.device = torch.device(device)
        self._c_cfg = c_config(cfg)
        self._keep = []
        w = dflash_weights()

        def arr(name):
            if name not in weights:
                return None
            ptrs = (c_void_p * cfg.n_layers)(*[t.data_ptr() for t in weights[name]])
            self._keep.append(ptrs)
            return ctypes.cast(ptrs, PP)

        for name in ("embed", "lm_head", "fc", "fc_scales", "ctx_norm", "final_norm"):
            t = weights.get(name)
            setattr(w, name, None if t is None else t.data_ptr())
        for name in ("wqkv", "wo", "wgu", "wd", "ln_in", "ln_post", "q_norm", "k_norm"):
            setattr(w, name, arr(name))
            if name in ("wqkv", "wo", "wgu", "wd"):
                setattr(w, name + "_scales", arr(name + "_scales"))
        self._weights = weights
        self._c_w = w
        ctx = c_void_p()
        create = self.lib.dflash_create_target if target else self.lib.dflash_create
        _check("dflash_create_target" if target else "dflash_create",
               create(ctypes.byref(self._c_cfg), ctypes.byref(w), ctypes.byref(ctx)))
        self.ctx = ctx
        self.layout = state_layout(cfg)
        self.state = torch.empty(self.layout["total"], dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(workspace_bytes(cfg), dtype=torch.uint8, device=self.device)
        _check("dflash_bind", self.lib.dflash_bind(ctx, self.state.data_ptr(), self.workspace.data_ptr(), _stream()))

    def __del__(self):
        ctx = getattr(self, "ctx", None)
        if ctx is not None and ctx.value:
            self.lib.dflash_destroy(ctx)
            self.ctx = None

    # ---------------------------------------------------------------- entry points
    def reset(self, req: int, valid_from: int, pos: int):
        _check("dflash_reset", self.lib.dflash_reset(self.ctx, _stream(), req, valid_from, pos))

    def tap_stage(self, taps: Sequence[torch.Tensor], n_rows: int, row_stride: Optional[int] = None,
                  req_of_row: Optional[torch.Tensor] = None, pos_of_row: Optional[torch.Tensor] = None,
                  rows_per_req: int = 0, ptrs: Optional[Sequence[int]] = None):
        """taps: n_taps fp32 tensors whose first row is staged row 0 (or raw
        pointers in ``ptrs``); row_stride defaults to the tensors' row stride."""
        c = self.cfg
        width = c.hc_streams * c.tap_hidden
        from_tensors = ptrs is None
        if from_tensors:
            if len(taps) != c.n_taps:
                raise ValueError(f"taps: expected {c.n_taps} tensors (got {len(taps)})")
            for i, t in enumerate(taps):
                _need(t, f"taps[{i}]", torch.float32, min_rows=n_rows)
                if t.dim() != 2 or t.shape[1] < width or t.stride(1) != 1:
                    raise ValueError(f"taps[{i}] must be [rows, >= {width}] with unit column stride")
            ptrs = [t.data_ptr() for t in taps]
            if row_stride is None:
                row_stride = taps[0].stride(0)
            if any(t.stride(0) != row_stride for t in taps):
                raise ValueError("every tap tensor must have the row stride of the call")
        elif len(ptrs) != c.n_taps:
            raise ValueError(f"ptrs: expected {c.n_taps} pointers (got {len(ptrs)})")
        _need(req_of_row, "req_of_row", torch.int32, shape=(n_rows,), optional=True)
        _need(pos_of_row, "pos_of_row", torch.int32, shape=(n_rows,), optional=True)
        _on_device(taps=list(taps) if from_tensors else [], req_of_row=req_of_row,
                   pos_of_row=pos_of_row)
        arr = (c_void_p * len(ptrs))(*ptrs)
        _check("dflash_tap_stage", self.lib.dflash_tap_stage(
            self.ctx, _stream(), ctypes.cast(arr, PP), int(row_stride), int(n_rows), _ptr(req_of_row),
            _ptr(pos_of_row), int(rows_per_req)))

    def draft_block(self, block_tokens: torch.Tensor, k: int = 1, logits: Optional[torch.Tensor] = None,
                    ids: Optional[torch.Tensor] = None, vals: Optional[torch.Tensor] = None):
        R = block_tokens.shape[0]
        Bm1 = max(self.cfg.block - 1, 1)
        self._check_draft(block_tokens, self.cfg.block, k, logits, ids, vals)
        if ids is None:
            ids = torch.empty((R, Bm1, k), dtype=torch.int32, device=self.device)
        _check("dflash_draft_block", self.lib.dflash_draft_block(
            self.ctx, _stream(), block_tokens.data_ptr(), R, _ptr(logits), ids.data_ptr(), _ptr(vals), k))
        return ids

    def draft_block_noalloc(self, block_tokens: torch.Tensor, k: int = 1, logits: Optional[torch.Tensor] = None,
                            ids: Optional[torch.Tensor] = None, vals: Optional[torch.Tensor] = None):
        """draft_block through the allocation-free entry point (the library's static
        device scratch instead of the bound workspace)."""
        R = block_tokens.shape[0]
        Bm1 = max(self.cfg.block - 1, 1)
        self._check_draft(block_tokens, self.cfg.block, k, logits, ids, vals)
        if ids is None:
            ids = torch.empty((R, Bm1, k), dtype=torch.int32, device=self.device)
        _check("dflash_draft_block_noalloc", self.lib.dflash_draft_block_noalloc(
            self.ctx, _stream(), block_tokens.data_ptr(), R, _ptr(logits), ids.data_ptr(), _ptr(vals), k))
        return ids

    def draft_block_n(self, block_tokens: torch.Tensor, k: int = 1, logits: Optional[torch.Tensor] = None,
                      ids: Optional[torch.Tensor] = None, vals: Optional[torch.Tensor] = None):
        """draft_block with the block length of this call = block_tokens.shape[1]."""
        R, b = block_tokens.shape
        self._check_draft(block_tokens, b, k, logits, ids, vals)
        if ids is None:
            ids = torch.empty((R, max(b - 1, 1), k), dtype=torch.int32, device=self.device)
        _check("dflash_draft_block_n", self.lib.dflash_draft_block_n(
            self.ctx, _stream(), block_tokens.data_ptr(), R, int(b), _ptr(logits), ids.data_ptr(), _ptr(vals), k))
        return ids

    def _check_draft(self, block_tokens, b, k, logits, ids, vals):
        if not isinstance(block_tokens, torch.Tensor) or block_tokens.dim() != 2:
            raise ValueError("block_tokens must be an int32 tensor [R, block]")
        R = block_tokens.shape[0]
        _need(block_tokens, "block_tokens", torch.int32, shape=(R, b))
        bm1 = max(b - 1, 1)
        _need(logits, "logits", torch.float32, shape=(R, bm1, self.cfg.vocab), optional=True)
        _need(ids, "ids", torch.int32, shape=(R, bm1, k), optional=True)
        _need(vals, "vals", torch.float32, shape=(R, bm1, k), optional=True)
        _on_device(block_tokens=block_tokens, logits=logits, ids=ids, vals=vals)

    def _check_accept(self, draft_ids, draft_stride, verify_ids, b, budget, out):
        if not isinstance(verify_ids, torch.Tensor) or verify_ids.dim() != 2:
            raise ValueError("verify_ids must be an int32 tensor [R, block]")
        R = verify_ids.shape[0]
        _need(verify_ids, "verify_ids", torch.int32, shape=(R, b))
        self._check_drafts(draft_ids, draft_stride, R, b, budget)
        if out is not None:
            _need(out.get("accept_len"), "out['accept_len']", torch.int32, shape=(R,))
            _need(out.get("emitted"), "out['emitted']", torch.int32, shape=(R, b))
            _need(out.get("n_emit"), "out['n_emit']", torch.int32, shape=(R,))
            _need(out.get("next_tokens"), "out['next_tokens']", torch.int32, shape=(R, b), optional=True)
        _on_device(verify_ids=verify_ids, draft_ids=draft_ids, budget=budget,
                   out=[] if out is None else [v for v in out.values() if v is not None])

    def _check_drafts(self, draft_ids, draft_stride, R, b, budget):
        if b > 1 or draft_ids is not None:
            # element (r, j) at (r * (b-1) + j) * draft_stride: [R, b-1] for stride 1, or
            # [R, b-1, k] top-k ids with stride k
            n = R * max(b - 1, 1) * int(draft_stride)
            _need(draft_ids, "draft_ids", torch.int32)
            if draft_ids.numel() != n or not draft_ids.is_contiguous() or draft_ids.shape[0] != R:
                raise ValueError(f"draft_ids must be a dense [{R}, {max(b - 1, 1)}(, {draft_stride})] tensor "
                                 f"(got {tuple(draft_ids.shape)})")
        _need(budget, "budget", torch.int32, shape=(R,), optional=True)

    def accept(self, draft_ids: torch.Tensor, draft_stride: int, verify_ids: torch.Tensor, eos_id: int = -1,
               budget: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None):
        B = self.cfg.block
        self._check_accept(draft_ids, draft_stride, verify_ids, B, budget, out)
        R = verify_ids.shape[0]
        if out is None:
            out = {"accept_len": torch.empty(R, dtype=torch.int32, device=self.device),
                   "emitted": torch.empty((R, B), dtype=torch.int32, device=self.device),
                   "n_emit": torch.empty(R, dtype=torch.int32, device=self.device),
                   "next_tokens": torch.empty((R, B), dtype=torch.int32, device=self.device)}
        _check("dflash_accept", self.lib.dflash_accept(
            self.ctx, _stream(), _ptr(draft_ids), int(draft_stride), verify_ids.data_ptr(), R, int(eos_id),
            _ptr(budget), out["accept_len"].data_ptr(), out["emitted"].data_ptr(), out["n_emit"].data_ptr(),
            _ptr(out.get("next_tokens"))))
        return out

    def accept_n(self, draft_ids: Optional[torch.Tensor], draft_stride: int, verify_ids: torch.Tensor,
                 eos_id: int = -1, budget: Optional[torch.Tensor] = None):
        """accept for a round of block length verify_ids.shape[1]."""
        R, b = verify_ids.shape
        self._check_accept(draft_ids, draft_stride, verify_ids, b, budget, None)
        out = {"accept_len": torch.empty(R, dtype=torch.int32, device=self.device),
               "emitted": torch.empty((R, b), dtype=torch.int32, device=self.device),
               "n_emit": torch.empty(R, dtype=torch.int32, device=self.device),
               "next_tokens": torch.empty((R, b), dtype=torch.int32, device=self.device)}
        _check("dflash_accept_n", self.lib.dflash_accept_n(
            self.ctx, _stream(), _ptr(draft_ids), int(draft_stride), verify_ids.data_ptr(), R, int(b), int(eos_id),
            _ptr(budget), out["accept_len"].data_ptr(), out["emitted"].data_ptr(), out["n_emit"].data_ptr(),
            out["next_tokens"].data_ptr()))
        return out

    def verify_block(self, block_tokens: torch.Tensor, tap_layers: Sequence[int] = (),
                     tap_out: Sequence[torch.Tensor] = (), logits: Optional[torch.Tensor] = None):
        """Verify pass of a target handle: argmax ids [R, b]; the residual rows after
        the tapped layers are written into tap_out (fp32 [R*b, >= hidden])."""
        R, b = block_tokens.shape
        _need(block_tokens, "block_tokens", torch.int32, shape=(R, b))
        _need(logits, "logits", torch.float32, shape=(R, b, self.cfg.vocab), optional=True)
        if len(tap_out) != len(tap_layers):
            raise ValueError("tap_out and tap_layers must have the same length")
        for i, t in enumerate(tap_out):
            _need(t, f"tap_out[{i}]", torch.float32, min_rows=R * b)
            if t.dim() != 2 or t.shape[1] < self.cfg.hidden or t.stride(1) != 1 or t.stride(0) != tap_out[0].stride(0):
                raise ValueError(f"tap_out[{i}] must be [rows, >= hidden] with one row pitch for all taps")
        _on_device(block_tokens=block_tokens, logits=logits, tap_out=list(tap_out))
        ids = torch.empty((R, b), dtype=torch.int32, device=self.device)
        n = len(tap_layers)
        layers = (ctypes.c_int * max(n, 1))(*tap_layers)
        outs = (c_void_p * max(n, 1))(*[t.data_ptr() for t in tap_out])
        ld = tap_out[0].stride(0) if n else 0
        _check("dflash_verify_block", self.lib.dflash_verify_block(
            self.ctx, _stream(), block_tokens.data_ptr(), R, int(b), ctypes.cast(layers, c_void_p) if n else None, n,
            ctypes.cast(outs, PP) if n else None, int(ld), _ptr(logits), ids.data_ptr()))
        return ids

    def accept_sampled(self, draft_ids: Optional[torch.Tensor], draft_stride: int, target_logits: torch.Tensor,
                       temperature: float = 1.0, top_k: int = 20, top_p: float = 0.95, eps: float = 0.2,
                       delta: float = 0.0, seed: int = 0, round: int = 0, eos_id: int = -1,
                       budget: Optional[torch.Tensor] = None):
        """Sampling-mode accept of a round of block length target_logits.shape[1]."""
        if not isinstance(target_logits, torch.Tensor) or target_logits.dim() != 3:
            raise ValueError("target_logits must be a float32 tensor [R, block, vocab]")
        R, b, _ = target_logits.shape
        _need(target_logits, "target_logits", torch.float32, shape=(R, b, self.cfg.vocab))
        self._check_drafts(draft_ids, draft_stride, R, b, budget)
        _on_device(target_logits=target_logits, draft_ids=draft_ids, budget=budget)
        out = {"accept_len": torch.empty(R, dtype=torch.int32, device=self.device),
               "emitted": torch.empty((R, b), dtype=torch.int32, device=self.device),
               "n_emit": torch.empty(R, dtype=torch.int32, device=self.device),
               "next_tokens": torch.empty((R, b), dtype=torch.int32, device=self.device)}
        prm = dflash_sampling(float(temperature), int(top_k), float(top_p), float(eps), float(delta))
        _check("dflash_accept_sampled", self.lib.dflash_accept_sampled(
            self.ctx, _stream(), _ptr(draft_ids), int(draft_stride), target_logits.data_ptr(), R, int(b),
            ctypes.byref(prm), int(seed) & (2 ** 64 - 1), int(round) & 0xFFFFFFFF, int(eos_id), _ptr(budget),
            out["accept_len"].data_ptr(), out["emitted"].data_ptr(), out["n_emit"].data_ptr(),
            out["next_tokens"].data_ptr()))
        return out

    # ---------------------------------------------------------------- candidate trees
    def tree_build(self, block_tokens: torch.Tensor, ids: torch.Tensor, vals: torch.Tensor, n_nodes: int):
        """(tokens, parent, depth) int32 [R, n_nodes] of the candidate trees built from
        the draft's top-k ids/values [R, block-1, k]."""
        R, B = block_tokens.shape
        k = ids.shape[-1]
        _need(block_tokens, "block_tokens", torch.int32, shape=(R, self.cfg.block))
        _need(ids, "ids", torch.int32, shape=(R, self.cfg.block - 1, k))
        _need(vals, "vals", torch.float32, shape=(R, self.cfg.block - 1, k))
        _on_device(block_tokens=block_tokens, ids=ids, vals=vals)
        out = [torch.empty((R, n_nodes), dtype=torch.int32, device=self.device) for _ in range(3)]
        _check("dflash_tree_build", self.lib.dflash_tree_build(
            self.ctx, _stream(), block_tokens.data_ptr(), ids.data_ptr(), vals.data_ptr(), int(k), R, int(n_nodes),
            *[t.data_ptr() for t in out]))
        return tuple(out)

    def verify_tree(self, tokens: torch.Tensor, parent: torch.Tensor, depth: torch.Tensor,
                    tap_layers: Sequence[int] = (), tap_out: Sequence[torch.Tensor] = (),
                    logits: Optional[torch.Tensor] = None):
        """Tree-masked verify pass of a target handle: ids [R, n] (each node's greedy next token)."""
        R, n = tokens.shape
        for name, t in (("tokens", tokens), ("parent", parent), ("depth", depth)):
            _need(t, name, torch.int32, shape=(R, n))
        _need(logits, "logits", torch.float32, shape=(R, n, self.cfg.vocab), optional=True)
        if len(tap_out) != len(tap_layers):
            raise ValueError("tap_out and tap_layers must have the same length")
        for i, t in enumerate(tap_out):
            _need(t, f"tap_out[{i}]", torch.float32, min_rows=R * n)
            if t.dim() != 2 or t.shape[1] < self.cfg.hidden or t.stride(1) != 1 or t.stride(0) != tap_out[0].stride(0):
                raise ValueError(f"tap_out[{i}] must be [rows, >= hidden] with one row pitch for all taps")
        _on_device(tokens=tokens, parent=parent, depth=depth, logits=logits, tap_out=list(tap_out))
        ids = torch.empty((R, n), dtype=torch.int32, device=self.device)
        m = len(tap_layers)
        layers = (ctypes.c_int * max(m, 1))(*tap_layers)
        outs = (c_void_p * max(m, 1))(*[t.data_ptr() for t in tap_out])
        ld = tap_out[0].stride(0) if m else 0
        _check("dflash_verify_tree", self.lib.dflash_verify_tree(
            self.ctx, _stream(), tokens.data_ptr(), parent.data_ptr(), depth.data_ptr(), R, int(n),
            ctypes.cast(layers, c_void_p) if m else None, m, ctypes.cast(outs, PP) if m else None, int(ld),
            _ptr(logits), ids.data_ptr()))
        return ids

    def tree_accept(self, tokens: torch.Tensor, parent: torch.Tensor, verify_ids: torch.Tensor, eos_id: int = -1,
                    budget: Optional[torch.Tensor] = None):
        """Tree accept on a drafter handle; returns the outputs of dflash_tree_accept."""
        R, n = tokens.shape
        B = self.cfg.block
        for name, t in (("tokens", tokens), ("parent", parent), ("verify_ids", verify_ids)):
            _need(t, name, torch.int32, shape=(R, n))
        _need(budget, "budget", torch.int32, shape=(R,), optional=True)
        _on_device(tokens=tokens, parent=parent, verify_ids=verify_ids, budget=budget)
        out = {"accept_len": torch.empty(R, dtype=torch.int32, device=self.device),
               "n_emit": torch.empty(R, dtype=torch.int32, device=self.device)}
        for name in ("emitted", "next_tokens", "path_nodes", "stage_rows", "stage_pos"):
            out[name] = torch.empty((R, B), dtype=torch.int32, device=self.device)
        _check("dflash_tree_accept", self.lib.dflash_tree_accept(
            self.ctx, _stream(), tokens.data_ptr(), parent.data_ptr(), int(n), verify_ids.data_ptr(), R, int(eos_id),
            _ptr(budget), out["accept_len"].data_ptr(), out["emitted"].data_ptr(), out["n_emit"].data_ptr(),
            out["next_tokens"].data_ptr(), out["path_nodes"].data_ptr(), out["stage_rows"].data_ptr(),
            out["stage_pos"].data_ptr()))
        return out

    def tree_commit(self, path_nodes: torch.Tensor, n_emit: torch.Tensor):
        """Commit a target's tree pass (K/V of the committed nodes into place, pos += n_emit)."""
        R, ld = path_nodes.shape
        _need(path_nodes, "path_nodes", torch.int32, shape=(R, ld))
        _need(n_emit, "n_emit", torch.int32, shape=(R,))
        _on_device(path_nodes=path_nodes, n_emit=n_emit)
        _check("dflash_tree_commit", self.lib.dflash_tree_commit(
            self.ctx, _stream(), path_nodes.data_ptr(), int(ld), n_emit.data_ptr(), R))

    def tap_stage_rows(self, taps: Sequence[torch.Tensor], src_row: torch.Tensor, pos_of_row: torch.Tensor,
                       rows_per_req: int, req_of_row: Optional[torch.Tensor] = None):
        """Stage the tap rows src_row[m] of `taps` (e.g. a tree pass's committed nodes)."""
        c = self.cfg
        n_rows = src_row.numel()
        if len(taps) != c.n_taps:
            raise ValueError(f"taps: expected {c.n_taps} tensors (got {len(taps)})")
        for i, t in enumerate(taps):
            _need(t, f"taps[{i}]", torch.float32)
            if t.dim() != 2 or t.shape[1] < c.hc_streams * c.tap_hidden or t.stride(1) != 1 or \
                    t.stride(0) != taps[0].stride(0):
                raise ValueError(f"taps[{i}] must be [rows, >= {c.hc_streams * c.tap_hidden}] with one row pitch")
        _need(src_row, "src_row", torch.int32, shape=(n_rows,))
        _need(pos_of_row, "pos_of_row", torch.int32, shape=(n_rows,))
        _need(req_of_row, "req_of_row", torch.int32, shape=(n_rows,), optional=True)
        _on_device(taps=list(taps), src_row=src_row, pos_of_row=pos_of_row, req_of_row=req_of_row)
        arr = (c_void_p * len(taps))(*[t.data_ptr() for t in taps])
        _check("dflash_tap_stage_rows", self.lib.dflash_tap_stage_rows(
            self.ctx, _stream(), ctypes.cast(arr, PP), int(taps[0].stride(0)), int(n_rows), src_row.data_ptr(),
            _ptr(req_of_row), pos_of_row.data_ptr(), int(rows_per_req)))

    def advance(self, n_emit: torch.Tensor):
        _need(n_emit, "n_emit", torch.int32, shape=(n_emit.numel(),) if isinstance(n_emit, torch.Tensor) else None)
        _on_device(n_emit=n_emit)
        _check("dflash_advance", self.lib.dflash_advance(self.ctx, _stream(), n_emit.data_ptr(), n_emit.numel()))

    def check(self) -> int:
        word = c_uint(0)
        rc = self.lib.dflash_check(self.ctx, _stream(), ctypes.byref(word))
        if rc not in (0, -7):
            _check("dflash_check", rc)
        return int(word.value)

    def clear_error(self):
        _check("dflash_clear_error", self.lib.dflash_clear_error(self.ctx, _stream()))

    def set_timing_events(self, kclass: int, before: Sequence, after: Sequence):
        n = len(before)
        b = (c_void_p * max(n, 1))(*[e.cuda_event if hasattr(e, "cuda_event") else e for e in before])
        a = (c_void_p * max(n, 1))(*[e.cuda_event if hasattr(e, "cuda_event") else e for e in after])
        self._keep.append((b, a))
        _check("dflash_set_timing_events", self.lib.dflash_set_timing_events(
            self.ctx, kclass, ctypes.cast(b, PP), ctypes.cast(a, PP), n))

    # ---------------------------------------------------------------- state views
    def positions(self):
        L, R = self.layout, self.cfg.max_requests
        pos = self.state[L["pos"]:L["pos"] + 4 * R].view(torch.int32)
        vf = self.state[L["valid_from"]:L["valid_from"] + 4 * R].view(torch.int32)
        return pos, vf

    def stats(self) -> torch.Tensor:
        L = self.layout
        n = self.cfg.block + 2
        return self.state[L["stats"]:L["stats"] + 8 * n].view(torch.int64)

    def ring(self):
        """(K [L, Rmax, nkv, C, hd], V^T [L, Rmax, nkv, hd, C]) bf16 views."""
        c, L = self.cfg, self.layout
        n = c.n_layers * c.max_requests * c.n_kv_heads * c.ring_capacity * c.head_dim
        k = self.state[L["ring_k"]:L["ring_k"] + 2 * n].view(torch.bfloat16).view(
            c.n_layers, c.max_requests, c.n_kv_heads, c.ring_capacity, c.head_dim)
        v = self.state[L["ring_v"]:L["ring_v"] + 2 * n].view(torch.bfloat16).view(
            c.n_layers, c.max_requests, c.n_kv_heads, c.head_dim, c.ring_capacity)
        return k, v


class BlockPolicy:
    """The library's adaptive block-length policy for one request (host code)."""

    def __init__(self, block: int, weight: float = 0.5):
        self.lib = load()
        self.p = dflash_block_policy()
        self.lib.dflash_policy_init(ctypes.byref(self.p), int(block), float(weight))

    def next_block(self) -> int:
        return int(self.lib.dflash_policy_next(ctypes.byref(self.p)))

    def update(self, accepted: int):
        self.lib.dflash_policy_update(ctypes.byref(self.p), int(accepted))

    @property
    def mean(self) -> float:
        return float(self.p.mean)
