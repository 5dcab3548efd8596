"""Helpers of the GPU parity tests: device copies of generated sessions and
the acceptance rules of the decode step.

Acceptance (scores are fp32 on the GPU, fp64-rounded-once in the oracle):
  * selection: with T the oracle's k-th score and B = {j : |s_j - T| <=
    1e-6 |T|}, the GPU's selection and the oracle's agree outside B, and the
    GPU selects exactly k_eff distinct valid rows;
  * attention: max |out_gpu - out_ref| <= 1e-3 max |out_ref|, where out_ref is
    the oracle's attention over the GPU's own selection.
"""
from __future__ import annotations

import numpy as np
import torch

SEL_BAND = 1e-6
ATTN_TOL = 1e-3
KEYS = ("idx_rows", "kv_rows", "q_idx", "w_idx", "q_attn")


def to_dev(s: dict, dev="cuda") -> dict:
    return {k: torch.from_numpy(np.ascontiguousarray(s[k])).to(dev) for k in KEYS}


def check_selection(gpu_sel: np.ndarray, ref_sel: np.ndarray, ref_scores_all: np.ndarray, k_eff: int) -> dict:
    """Set equality outside the band around the oracle's k-th score."""
    g = [int(x) for x in gpu_sel[:k_eff]]
    assert all(x == -1 for x in gpu_sel[k_eff:]), "padding must be -1"
    assert len(set(g)) == k_eff and all(0 <= x < len(ref_scores_all) for x in g), "k_eff distinct valid rows"
    if k_eff == 0:
        return {"band": 0, "swaps": 0}
    T = float(ref_scores_all[ref_sel[k_eff - 1]])
    band = np.abs(ref_scores_all.astype(np.float64) - T) <= SEL_BAND * abs(T)
    diff = set(g) ^ set(int(x) for x in ref_sel[:k_eff])
    outside = sorted(j for j in diff if not band[j])
    assert not outside, f"selection differs outside the band at rows {outside[:10]}"
    return {"band": int(band.sum()), "swaps": len(diff) // 2}


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
