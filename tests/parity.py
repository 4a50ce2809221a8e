"""Shared parity rules for GPU-vs-oracle checks.

Tolerances (floating point): per-key scores within relative 1e-3 of the fp64
oracle, the row normalisers m within 1e-4 + 1e-5*|m| and Z within relative
1e-4. Index sets must match exactly outside the tie band of each head; the
gather is compared bit for bit.
"""
from __future__ import annotations

import numpy as np

import oracle

SCORE_RTOL = 1e-3
M_ATOL = 1e-4
M_RTOL = 1e-5
Z_RTOL = 1e-4


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return np.abs(got - want) / np.maximum(np.abs(want), 1e-300)


def assert_scores_close(got, want, rtol=SCORE_RTOL, what="scores"):
    err = rel_err(got, want)
    # Scores below 1e-30 are compared absolutely (far below anything that can rank).
    tiny = np.abs(want) < 1e-30
    err = np.where(tiny, np.abs(np.asarray(got, np.float64) - want), err)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= rtol, f"{what}: max relative error {worst:.3e} > {rtol:.1e}"
    return worst


def assert_normalizers_close(m_got, z_got, m_want, z_want):
    m_got = np.asarray(m_got, np.float64)
    dm = np.abs(m_got - m_want)
    lim = M_ATOL + M_RTOL * np.abs(m_want)
    assert np.all(dm <= lim), f"m: max abs error {dm.max():.3e}"
    zr = rel_err(z_got, z_want)
    assert zr.max() <= Z_RTOL, f"Z: max relative error {zr.max():.3e}"


def tie_band(values: np.ndarray, budget: int, n_sink: int, n_recent: int, eps: float):
    """Keys whose oracle value lies within the band where a relative error of
    eps on every value can swap their order with the threshold: with tau the
    k_sel-th best candidate value, {j : tau(1-eps)/(1+eps) <= v_j <= tau(1+eps)/(1-eps)}."""
    s = values.shape[0]
    if budget >= s:
        return np.zeros(0, dtype=np.int64)
    mand = oracle.mandatory(s, n_sink, n_recent)
    is_cand = np.ones(s, dtype=bool)
    is_cand[mand] = False
    cand = np.nonzero(is_cand)[0]
    k_sel = budget - mand.size
    if k_sel <= 0 or cand.size == 0:
        return np.zeros(0, dtype=np.int64)
    tau = np.sort(values[cand])[::-1][k_sel - 1]
    lo, hi = tau * (1 - eps) / (1 + eps), tau * (1 + eps) / (1 - eps)
    band = cand[(values[cand] >= lo) & (values[cand] <= hi)]
    return band


def assert_selection_matches(gpu_idx: np.ndarray, oracle_idx: np.ndarray, values: np.ndarray,
                             budget: int, n_sink: int, n_recent: int, eps: float = SCORE_RTOL):
    """Index-set parity of one head: same size, ascending, mandatory keys kept,
    and any difference lies inside the tie band. Returns the band size."""
    s = values.shape[0]
    want_n = min(budget, s)
    assert gpu_idx.shape == (want_n,), f"retained {gpu_idx.shape[0]} keys, want {want_n}"
    assert np.all(np.diff(gpu_idx) > 0), "indices not strictly ascending"
    assert gpu_idx.min() >= 0 and gpu_idx.max() < s
    mand = oracle.mandatory(s, n_sink, n_recent) if budget < s else np.arange(s)
    assert np.isin(mand, gpu_idx).all(), "a mandatory key is missing"
    diff = np.setxor1d(gpu_idx, oracle_idx)
    band = tie_band(values, budget, n_sink, n_recent, eps)
    outside = np.setdiff1d(diff, band)
    assert outside.size == 0, f"{outside.size} keys differ outside the tie band (|band|={band.size})"
    return band.size


def assert_selection_consistent(gpu_idx: np.ndarray, gpu_vals: np.ndarray, budget: int,
                                n_sink: int, n_recent: int):
    """The GPU's own choice is an exact top-k of the GPU's own values under
    (value desc, index asc): checks what is unique at any size."""
    s = gpu_vals.shape[0]
    want = oracle.select_head(gpu_vals.astype(np.float64), budget, n_sink, n_recent)
    np.testing.assert_array_equal(gpu_idx, want)
