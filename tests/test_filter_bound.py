"""The filter's bound, checked on the CPU.

The decode step scores rows with the query held to three fp6 (E2M3) terms per
32-value block and brackets each row's exact score by

    beta_j = sum_b Z_b 2^(s_jb - 127) + Z_abs,
    Z_b = 6 (1 + 2^-10) sum_h |w_h| (rho_hb + 2^-15 A_hb),  Z_abs = 2^-117 sum_h |w_h|,

rho_hb = L1 norm of the query residual of head h in block b, A_hb = an upper
bound on the L1 norm of the terms plus rho_hb: the kernel takes
A_hb = sum |q| + sum_t 2^(E_t + 4) over the block's term exponents E_t
(csa_score.hpp, csa_bound.hpp).  Here the split is emulated in numpy
(the same exponent rule, round-to-nearest-even onto the E2M3 grid) and the
bound is checked against exact arithmetic on adversarial queries:

  * the split is exact: q = t0 + t1 + t2 + r, and |r| <= max(2^-11.9 max|q|,
    2^-130) per block (the floor: term scales stop at 2^-126);
  * the kernel's closed-form A_hb is at least the exact L1 norm of the terms
    plus the residual;
  * the filter's score with exact sums, s~ = sum_h w_h max(0, (t0+t1+t2)_h . k),
    lies within the residual part of beta of the exact score, and the oracle's
    fp32 score lies within beta of s~;
  * the residual part is not vacuous: on rows built to align the residual
    with the row's codes, the error reaches a fixed fraction of it.

The GPU's own filter is checked against its brackets in test_gpu_parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest

import pins

F32_MAX = float(np.finfo(np.float32).max)


def e2m3_rne(y: np.ndarray) -> np.ndarray:
    """Round to the E2M3 grid (magnitudes 0..7.5: spacing 1/8 below 2, 1/4 in
    [2, 4), 1/2 in [4, 8)), ties to even, saturating at 7.5."""
    mag = np.abs(y)
    step = np.where(mag < 2.0, 0.125, np.where(mag < 4.0, 0.25, 0.5))
    q = np.round(mag / step) * step  # numpy rounds half to even
    q = np.minimum(q, 7.5)
    return np.copysign(q, y)


def split_block(x: np.ndarray, terms: int = 3):
    """Split one 32-value fp32 block as the kernel does; returns (terms,
    residual) in float64 (all exact)."""
    x = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x)))
    ab = int(amax.view(np.uint32))
    E0 = (ab >> 23) - 129 + (1 if (ab & 0x7FFFFF) > 0x700000 else 0)
    E0 = 0 if amax == 0 else E0
    E0 = min(max(E0, -126), 127)
    r = x.astype(np.float64)
    out = []
    exps = []
    for t in range(terms):
        E = max(E0 - 4 * t, -126)
        qt = e2m3_rne(r / 2.0**E) * 2.0**E
        out.append(qt)
        exps.append(E)
        r = r - qt
    split_block.exps = exps
    return out, r


def adversarial_query(rng, h: int) -> np.ndarray:
    q = rng.standard_normal((h, 128)).astype(np.float32)
    for hh in range(h):
        kind = hh % 6
        if kind == 1:  # one huge value per block, the rest tiny: large in-block dynamic range
            q[hh] *= np.float32(1e-4)
            q[hh, rng.integers(0, 32, 4) + 32 * np.arange(4)] = np.float32(3e4) * rng.choice([-1, 1], 4)
        elif kind == 2:  # values spread over 60 binades
            q[hh] = (rng.choice([-1, 1], 128) * 2.0 ** rng.uniform(-30, 30, 128)).astype(np.float32)
        elif kind == 3:  # subnormal and zero blocks
            q[hh, :32] = 0.0
            q[hh, 32:64] = (rng.integers(-2**20, 2**20, 32) * 2.0**-149).astype(np.float32)
        elif kind == 4:  # values just below the E2M3 rounding ties
            q[hh] = (rng.integers(1, 60, 128) * 0.125 + 0.0624).astype(np.float32) * rng.choice([-1, 1], 128)
        elif kind == 5:  # a huge head
            q[hh] *= np.float32(2.0**40)
    return q


def bound_constants(q: np.ndarray, w: np.ndarray):
    h = q.shape[0]
    rho = np.zeros((h, 4))
    mag = np.zeros((h, 4))
    qt_sum = np.zeros((h, 128))
    for hh in range(h):
        for b in range(4):
            terms, r = split_block(q[hh, 32 * b:32 * b + 32])
            t_sum = sum(terms)
            # the split is exact: q = sum of terms + r
            assert np.array_equal(t_sum + r, q[hh, 32 * b:32 * b + 32].astype(np.float64))
            amax = float(np.max(np.abs(q[hh, 32 * b:32 * b + 32])))
            # relative to the block's largest value, floored at half the
            # finest term spacing (scales clamp at 2^-126: subnormal blocks)
            assert np.max(np.abs(r)) <= max(2.0**-11.9 * amax, 2.0**-130)
            rho[hh, b] = np.sum(np.abs(r))
            exact_mag = sum(np.sum(np.abs(t)) for t in terms) + rho[hh, b]
            # the kernel's closed form, an upper bound on that norm
            mag[hh, b] = np.sum(np.abs(q[hh, 32 * b:32 * b + 32].astype(np.float64))) + sum(
                2.0 ** (E + 4) for E in split_block.exps)
            assert mag[hh, b] >= exact_mag
            qt_sum[hh, 32 * b:32 * b + 32] = t_sum
    wa = np.abs(w.astype(np.float64))
    z_res = 6.0 * (wa[:, None] * rho).sum(axis=0)                      # residual part, per block
    z = 6.0 * (1 + 2.0**-10) * (wa[:, None] * (rho + 2.0**-15 * mag)).sum(axis=0)
    zabs = 2.0**-117 * wa.sum()
    return qt_sum, z_res, z, zabs


def rows_with_scales(rng, n: int) -> np.ndarray:
    rows = pins.random_idx_rows(n, int(rng.integers(1 << 30)))
    a, b = n // 3, 2 * n // 3
    rows[:a, 64:68] = rng.integers(0, 253, size=(a, 4))         # any scale byte that decodes finitely
    rows[a:b, 64:68] = rng.integers(118, 136, size=(b - a, 4))  # the usual range
    rows[b:, 64:68] = rng.integers(0, 8, size=(n - b, 4))       # tiny scales: subnormal values
    return rows


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_bracket_holds_on_adversarial_queries(orc, seed):
    rng = np.random.default_rng(seed)
    h = 12
    q = adversarial_query(rng, h)
    w = (rng.uniform(-1, 1, h) * 2.0 ** rng.integers(-20, 20, h)).astype(np.float32)
    rows = rows_with_scales(rng, 600)
    k = pins.ref_decode_idx(rows).astype(np.float64)
    assert np.all(np.isfinite(k))
    qt, z_res, z, zabs = bound_constants(q, w)
    S = orc.score(rows, q, w).astype(np.float64)                       # the oracle's fp32 scores
    d = k @ q.astype(np.float64).T
    s_exact = (w.astype(np.float64)[None, :] * np.maximum(d, 0)).sum(axis=1)
    s_filt = (w.astype(np.float64)[None, :] * np.maximum(k @ qt.T, 0)).sum(axis=1)
    scale = 2.0 ** (rows[:, 64:68].astype(np.float64) - 127)
    beta_res = scale @ z_res
    beta = scale @ z + zabs
    ok = np.isfinite(s_exact) & (np.abs(s_exact) < F32_MAX)
    # the residual part bounds the filter's distance from the exact score
    # (up to the fp64 rounding of these sums, far below it)
    assert np.all(np.abs(s_filt - s_exact)[ok] <= beta_res[ok] * (1 + 1e-9) + 1e-300)
    # the whole bound brackets the oracle's fp32 score around the filter score
    assert np.all(np.abs(S - s_filt)[ok] <= beta[ok])


def test_bracket_residual_term_is_tight():
    """A row whose codes all have magnitude 6 and the residual's signs: the
    residual term then equals the error (the bound is reached)."""
    rng = np.random.default_rng(5)
    q = adversarial_query(rng, 1)
    w = np.ones(1, np.float32)
    qt, z_res, _, _ = bound_constants(q, w)
    r = q.astype(np.float64)[0] - qt[0]
    codes = np.where(r >= 0, 7, 15)  # +6 / -6 in E2M1
    row = np.zeros(68, np.uint8)
    row[:64] = codes[0::2] | (codes[1::2] << 4)
    row[64:68] = 127
    k = pins.ref_decode_idx(row[None])[0].astype(np.float64)
    err = abs(float(r @ k))
    assert err == pytest.approx(float(z_res.sum()), rel=1e-12)
