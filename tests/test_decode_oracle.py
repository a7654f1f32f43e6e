"""Decode-time rescoring in the oracle (CPU).

Pins: after any number of appended tokens, the incrementally maintained raw
score equals the score of the grown cache computed from its definition
(the closed form, itself pinned to delete-and-recompute elsewhere), and on
tiny caches equals the literal delete-and-recompute of the final window;
re-eviction on the maintained score equals prefill eviction of the grown
cache; a singular new row is rejected.
"""

import numpy as np
import pytest

import oracle
from oracle.decode import decode_init, decode_scratch, decode_select, decode_step
from brute_force import brute_force_scores


def _cache(seed, Hq, Hkv, d, n_total, w):
    rng = np.random.default_rng(seed)
    q_all = rng.standard_normal((Hq, n_total, d))  # query rows of every position
    k = rng.standard_normal((Hkv, n_total, d)) * 1.3
    v = rng.standard_normal((Hkv, n_total, d))
    return q_all, k, v


def _run(seed, Hq, Hkv, d, n0, w, steps):
    q_all, k, v = _cache(seed, Hq, Hkv, d, n0 + steps, w)
    st = decode_init(q_all[:, n0 - w:n0], k, v, n=n0, window=w, Hq=Hq, Hkv=Hkv, d=d)
    for s in range(steps):
        st = decode_step(st, q_all[:, n0 + s], k, v)
    return st, q_all, k, v


@pytest.mark.parametrize("seed,Hq,Hkv,d,n0,w,steps", [
    (0, 4, 2, 8, 20, 3, 7),     # every window row of the prefill leaves, then new ones do
    (1, 2, 2, 16, 12, 1, 5),    # window of one row, one query head per KV head
    (2, 8, 2, 8, 30, 6, 9),     # G = 4
    (3, 7, 1, 8, 25, 4, 4),     # G = 7, steps == window
])
def test_incremental_equals_scratch(seed, Hq, Hkv, d, n0, w, steps):
    st, q_all, k, v = _run(seed, Hq, Hkv, d, n0, w, steps)
    n = n0 + steps
    assert st["n"] == n and st["S"].shape == (Hkv, n)
    np.testing.assert_array_equal(st["q_win"], q_all[:, n - w:n])
    ref = decode_scratch(q_all[:, n - w:n], k, v, n=n, window=w, Hq=Hq, Hkv=Hkv, d=d)
    err = np.abs(st["S"] - ref).max() / np.abs(ref).max()
    assert err < 1e-12, err
    # tokens appended after the window's oldest row still score only from the rows that see them
    assert np.all(st["S"] >= -1e-12 * np.abs(ref).max())


def test_incremental_equals_delete_and_recompute():
    Hq, Hkv, d, n0, w, steps = 4, 2, 4, 9, 3, 4
    st, q_all, k, v = _run(11, Hq, Hkv, d, n0, w, steps)
    n = n0 + steps
    _, S_bf = brute_force_scores(q_all[:, n - w:n], k[:, :n], v[:, :n], n, w, Hq, Hkv)
    np.testing.assert_allclose(st["S"], S_bf, rtol=1e-10, atol=1e-14)


def test_reevict_equals_prefill_eviction():
    Hq, Hkv, d, n0, w, steps = 4, 2, 8, 40, 5, 8
    st, q_all, k, v = _run(5, Hq, Hkv, d, n0, w, steps)
    n = n0 + steps
    sel = decode_select(st, pool_kernel=3, n_evict=17)
    ref = oracle.dropkv_oracle(q_all[:, n - w:n], k[:, :n], v[:, :n], n=n, window=w, Hq=Hq, Hkv=Hkv, d=d,
                               pool_kernel=3, n_evict=17, dtype="f64")
    fin = np.isfinite(ref["P"])
    np.testing.assert_array_equal(np.isfinite(sel["P"]), fin)
    np.testing.assert_allclose(sel["P"][fin], ref["P"][fin], rtol=1e-12)
    np.testing.assert_array_equal(sel["evict"], ref["evict"])


def test_step_rejects_singular_new_row():
    Hq, Hkv, d, n0, w = 2, 1, 8, 10, 2
    q_all, k, v = _cache(3, Hq, Hkv, d, n0 + 1, w)
    st = decode_init(q_all[:, n0 - w:n0], k, v, n=n0, window=w, Hq=Hq, Hkv=Hkv, d=d)
    q_new = q_all[:, n0].copy()
    k = k.copy()
    k[0, 4] = 200.0 * q_new[1] / np.linalg.norm(q_new[1])  # logit gap far beyond 2^-24 rest mass
    with pytest.raises(oracle.SingularRow):
        decode_step(st, q_new, k, v)
