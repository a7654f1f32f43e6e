"""CPU checks of the eviction-set rules the GPU parity tests apply (tests/parity.py).

Synthetic oracle scores with a pooling plateau at the boundary, and GPU
scores perturbed within a known relative error: the rules must accept every
consistent result and reject sets that are not the GPU's own bottom-k,
scores outside the tolerance, and a set that differs where the gap rule
demands equality.
"""

import numpy as np
import pytest

from parity import check_evictions, own_bottom_k, symdiff_band


def _ref(n=4000, w=16, seed=0):
    rng = np.random.default_rng(seed)
    S = rng.lognormal(size=(1, n))
    P = S.copy()
    P[0, 1000:1007] = P[0, 1003]  # a plateau copied bit for bit
    P[0, n - w:] = np.inf
    return S, P


def test_band_is_symmetric_in_ratio():
    lo, hi = symdiff_band(0.01)
    assert lo * hi == pytest.approx(1.0) and lo < 1.0 < hi
    assert hi - 1.0 == pytest.approx(2 * 0.01, rel=0.02)


@pytest.mark.parametrize("e", [1e-6, 1e-3, 1e-2])
def test_consistent_perturbations_pass(e):
    S, P = _ref()
    rng = np.random.default_rng(1)
    for k in (1, 500, 1003, 2000, 3984):
        gpu = P * (1 + rng.uniform(-e, e, size=P.shape))
        gpu[np.isinf(P)] = np.inf
        idx = own_bottom_k(gpu[0], k)[None, :]
        ref_idx = own_bottom_k(P[0], k)[None, :]
        rep = {}
        check_evictions(gpu, idx, P, S, ref_idx, k, 2e-2, report=rep)
        assert rep["gap_exact"] + rep["plateau_exact"] + rep["band_checked"] == 1


def test_not_own_bottom_k_is_rejected():
    S, P = _ref()
    k = 700
    idx = own_bottom_k(P[0], k).copy()
    idx[-1] = int(np.argmax(np.where(np.isinf(P[0]), -1, P[0])))  # the largest finite score
    idx = np.sort(idx)[None, :]
    with pytest.raises(AssertionError):
        check_evictions(P, idx, P, S, own_bottom_k(P[0], k)[None, :], k, 2e-2)


def test_error_beyond_tolerance_is_rejected():
    S, P = _ref()
    k = 1500
    ref_idx = own_bottom_k(P[0], k)
    gpu = P.copy()
    out = ref_idx[-1]            # the oracle's boundary token, scored 10% high on the GPU
    gpu[0, out] *= 1.10
    idx = own_bottom_k(gpu[0], k)[None, :]
    with pytest.raises(AssertionError):
        check_evictions(gpu, idx, P, S, ref_idx[None, :], k, 2e-2)


def test_gap_rule_demands_equality():
    n, w, k = 64, 4, 10
    S = np.arange(1, n + 1, dtype=np.float64)[None, :] * 10.0  # gaps of 10 / (10 k) >> 2 rtol
    P = S.copy()
    P[0, n - w:] = np.inf
    ref_idx = own_bottom_k(P[0], k)[None, :]
    rep = {}
    check_evictions(P, ref_idx, P, S, ref_idx, k, 2e-2, report=rep)
    assert rep["gap_exact"] == 1
    bad = P.copy()
    bad[0, k] = bad[0, k - 1] * 0.999   # GPU swaps the k-th and (k+1)-th: 10% error
    idx = own_bottom_k(bad[0], k)[None, :]
    with pytest.raises(AssertionError):
        check_evictions(bad, idx, P, S, ref_idx, k, 2e-2)
