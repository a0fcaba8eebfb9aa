"""Shared helpers of the GPU parity tests: inputs for both sides, tolerance and
top-k comparisons against the oracle."""
from __future__ import annotations

import numpy as np
import torch

from block_diffusion_drafter_tap_amd import synth


def host_weights(w):
    """fp32 numpy copies (exact) of the weights the GPU reads; INT4 matrices are
    left packed for the oracle's own unpacker."""
    out = {}
    for k, v in w.items():
        if isinstance(v, list):
            out[k] = [synth.bf16_to_f32_numpy(t) if t.dtype != torch.uint8 else t.cpu().numpy() for t in v]
        else:
            out[k] = synth.bf16_to_f32_numpy(v) if v.dtype != torch.uint8 else v.cpu().numpy()
    return out


def tol(ref: np.ndarray) -> float:
    """|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3 (bf16 in, fp32 accumulate)."""
    return 1e-2 * float(np.max(np.abs(ref))) + 1e-3


def assert_close(gpu, ref, what: str):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = float(np.max(np.abs(gpu - ref)))
    t = tol(ref)
    assert err <= t, f"{what}: max |gpu - oracle| = {err:.4g} > tol {t:.4g}"
    return err


def topk_self_consistent(gpu_logits: np.ndarray, gpu_ids: np.ndarray):
    """GPU ids must be exactly the (value desc, index asc) order of the GPU's own logits."""
    k = gpu_ids.shape[-1]
    L = gpu_logits.reshape(-1, gpu_logits.shape[-1])
    ids = gpu_ids.reshape(-1, k)
    for r in range(L.shape[0]):
        ref = np.lexsort((np.arange(L.shape[1]), -L[r].astype(np.float64)))[:k]
        np.testing.assert_array_equal(ids[r], ref, err_msg=f"row {r}")


def topk_valid_within_error(oracle_logits: np.ndarray, gpu_ids: np.ndarray, k: int, gpu_logits: np.ndarray):
    """Every rank of every GPU top-k list checked against the oracle, ties or not.

    With eps_row = max |gpu - oracle| over the row, an exact top-k of the GPU
    logits satisfies, for any rounding within eps_row: its ids are distinct and
    in range; each id's oracle logit is at least the oracle's k-th largest value
    minus 2 eps_row (the GPU's k-th largest is at least the oracle's minus eps_row);
    and consecutive ranks keep their oracle order up to 2 eps_row. A wrong or
    misplaced id fails one of these unless it lies within the error band. Returns
    the number of ranks checked."""
    L = np.asarray(oracle_logits, dtype=np.float64).reshape(-1, np.shape(oracle_logits)[-1])
    G = np.asarray(gpu_logits, dtype=np.float64).reshape(L.shape)
    ids = np.asarray(gpu_ids).reshape(-1, k)
    n = 0
    for r in range(L.shape[0]):
        sel = ids[r].astype(np.int64)
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < L.shape[1], f"row {r}: ids {sel}"
        band = 2.0 * float(np.max(np.abs(G[r] - L[r]))) + 1e-9 * (1.0 + float(np.max(np.abs(L[r]))))
        kth = np.partition(L[r], L.shape[1] - k)[L.shape[1] - k]
        v = L[r][sel]
        assert v.min() >= kth - band, f"row {r}: id {sel[np.argmin(v)]} oracle {v.min()} < k-th {kth} - {band}"
        for j in range(k - 1):
            assert v[j] >= v[j + 1] - band, f"row {r} ranks {j},{j + 1}: oracle {v[j]} < {v[j + 1]} - {band}"
        n += k
    return n


def topk_agrees_away_from_ties(oracle_logits: np.ndarray, gpu_ids: np.ndarray, k: int,
                               gpu_logits: np.ndarray = None):
    """Compare GPU ids with the oracle's at the ranks the numerics decide.

    Rank j of a row is compared when the oracle's gaps to ranks j-1 and j+1
    exceed delta = max(2 * eps_row, 1e-3 * max|row| + 1e-5), eps_row being the
    measured max |gpu - oracle| logit error of that row: if every GPU logit is
    within eps_row of the oracle's, two values more than 2 * eps_row apart keep
    their order, so a mismatch there is a selection bug, not rounding. Returns
    (compared, excluded) counts. Given the GPU logits, every rank is also checked
    by topk_valid_within_error."""
    L = oracle_logits.reshape(-1, oracle_logits.shape[-1])
    G = None if gpu_logits is None else np.asarray(gpu_logits, dtype=np.float64).reshape(L.shape)
    if G is not None:
        topk_valid_within_error(L, gpu_ids, k, G)
    ids = gpu_ids.reshape(-1, k)
    compared = excluded = 0
    for r in range(L.shape[0]):
        order = np.lexsort((np.arange(L.shape[1]), -L[r]))[:k + 1]
        v = L[r][order]
        delta = 1e-3 * np.max(np.abs(L[r])) + 1e-5
        if G is not None:
            delta = max(delta, 2.0 * float(np.max(np.abs(G[r] - L[r]))))
        for j in range(k):
            lo_gap = v[j - 1] - v[j] if j > 0 else np.inf
            hi_gap = v[j] - v[j + 1]
            if min(lo_gap, hi_gap) > delta:
                assert ids[r, j] == order[j], f"row {r} rank {j}: gpu {ids[r, j]} oracle {order[j]}"
                compared += 1
            else:
                excluded += 1
    return compared, excluded


def topk_within_eps(oracle_logits: np.ndarray, gpu_ids: np.ndarray, gpu_logits: np.ndarray):
    """Every rank, near-ties included: the oracle's logit of the id the GPU put at
    rank j lies within 2 * eps_row of the oracle's rank-j value, eps_row being the
    row's max |gpu - oracle| logit error. This holds for any correct selection
    (the GPU's rank-j value is its j-th largest logit, which is within eps_row of
    the oracle's j-th largest, and the GPU's logit of an id is within eps_row of
    the oracle's), so a wrong id anywhere in the list fails it unless it is a
    genuine near-tie. Returns the largest |difference| / (2 * eps_row) seen."""
    L = oracle_logits.reshape(-1, oracle_logits.shape[-1]).astype(np.float64)
    G = np.asarray(gpu_logits, dtype=np.float64).reshape(L.shape)
    k = gpu_ids.shape[-1]
    ids = gpu_ids.reshape(-1, k)
    worst = 0.0
    for r in range(L.shape[0]):
        eps = float(np.max(np.abs(G[r] - L[r])))
        v = np.sort(L[r])[::-1][:k]
        d = np.abs(L[r][ids[r]] - v)
        bound = 2.0 * eps + 1e-12
        assert np.all(d <= bound), f"row {r}: rank {int(np.argmax(d - bound))} off by {float(np.max(d)):.4g} > {bound:.4g}"
        worst = max(worst, float(np.max(d)) / bound)
    return worst


def require_compared(comp: int, excl: int, min_frac: float, what: str):
    """The tie-excluding comparison must still decide a stated share of ranks."""
    total = comp + excl
    frac = comp / max(total, 1)
    print(f"{what}: ranks compared {comp} of {total} ({frac:.0%}; minimum {min_frac:.0%}), near-ties excluded {excl}",
          flush=True)
    assert frac >= min_frac, f"{what}: only {comp} of {total} ranks decided by the numerics"
