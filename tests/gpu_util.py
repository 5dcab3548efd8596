"""Helpers of the GPU parity tests: device copies of generated sessions and
the acceptance rules of the decode step.

Acceptance:
  * selection: the GPU's selection is the oracle's, row for row and in the
    same order, and sel_score holds the oracle's scores bit for bit (the
    candidates are rescored exactly in the reference's fp64 arithmetic);
  * attention: max |out_gpu - out_ref| <= 1e-3 max |out_ref|, where out_ref is
    the oracle's attention over the GPU's own selection (lse within 1e-5).
"""
from __future__ import annotations

import numpy as np
import torch

ATTN_TOL = 1e-3
KEYS = ("idx_rows", "kv_rows", "q_idx", "w_idx", "q_attn")


def to_dev(s: dict, dev="cuda") -> dict:
    return {k: torch.from_numpy(np.ascontiguousarray(s[k])).to(dev) for k in KEYS}


def check_selection_exact(gpu_sel: np.ndarray, gpu_score: np.ndarray, ref_sel: np.ndarray, ref_score: np.ndarray,
                          k_eff: int) -> dict:
    """The GPU's selection is the oracle's: the same rows in the same order
    and the same scores bit for bit, -1 / -inf padded."""
    assert np.array_equal(gpu_sel, ref_sel), (
        f"selection differs at {int(np.sum(gpu_sel != ref_sel))} positions, first {np.nonzero(gpu_sel != ref_sel)[0][:5]}")
    g, r = gpu_score[:k_eff].astype(np.float32), ref_score[:k_eff].astype(np.float32)
    assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), "selected scores differ"
    assert np.all(np.isneginf(gpu_score[k_eff:]))
    return {"exact": True}


def check_attention(gpu_out: np.ndarray, ref_out: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref_out))) if ref_out.size else 0.0
    err = float(np.max(np.abs(gpu_out - ref_out))) if ref_out.size else 0.0
    if scale == 0.0:
        assert err == 0.0
        return 0.0
    rel = err / scale
    assert rel <= ATTN_TOL, f"attention error {rel:.3e} > {ATTN_TOL}"
    return rel


def topk_keys_host(scores: np.ndarray, k: int) -> np.ndarray:
    """Exact top-k rows of a score array by (score desc, row asc); NaN last."""
    s = scores.astype(np.float64)
    nan = np.isnan(s)
    neg = np.where(nan, 0.0, -s) + 0.0  # -0 ties +0
    order = np.lexsort((np.arange(len(s)), neg, nan.astype(np.int8)))
    return order[:k].astype(np.int32)
