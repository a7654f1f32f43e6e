"""Pins of the prefill-attention oracle (oracle/prefill.py) on the CPU.

Against things other than itself: a pure-Python softmax loop over the visible
keys (brute force), the one-key case (position 0 sees only key 0, so its
output is v_0 exactly), equal keys (uniform attention: the output is the mean
of the visible values), and the window rows' outputs from the scoring
oracle's row statistics (the same definition through another code path).
"""

import math

import numpy as np
import pytest

import oracle


def _case(seed, Hq=4, Hkv=2, d=8, n=20):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Hq, n, d)), rng.standard_normal((Hkv, n, d)) * 1.3,
            rng.standard_normal((Hkv, n, d)))


def _brute(q, k, v, h, pos, G):
    g = h // G
    d = q.shape[2]
    logits = [sum(q[h, pos, c] * k[g, j, c] for c in range(d)) / math.sqrt(d) for j in range(pos + 1)]
    top = max(logits)
    w = [math.exp(x - top) for x in logits]
    tot = math.fsum(w)
    return np.array([math.fsum(w[j] / tot * v[g, j, c] for j in range(pos + 1)) for c in range(d)])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_outputs_equal_brute_force(seed):
    q, k, v = _case(seed)
    Hq, Hkv, n = q.shape[0], k.shape[0], q.shape[1]
    rows = [(h, pos) for h in range(Hq) for pos in range(n)]
    out = oracle.prefill_outputs(q, k, v, rows, Hq=Hq, Hkv=Hkv)
    for r, (h, pos) in enumerate(rows):
        ref = _brute(q, k, v, h, pos, Hq // Hkv)
        assert np.max(np.abs(out[r] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_position_zero_sees_only_key_zero():
    q, k, v = _case(5)
    out = oracle.prefill_outputs(q, k, v, [(h, 0) for h in range(4)], Hq=4, Hkv=2)
    for h in range(4):
        assert np.array_equal(out[h], v[h // 2, 0])


def test_equal_keys_give_the_mean_of_visible_values():
    q, k, v = _case(6)
    k[:] = k[:, :1, :]  # every key of a head equal to its first
    rows = [(1, 7), (2, 13), (3, 19)]
    out = oracle.prefill_outputs(q, k, v, rows, Hq=4, Hkv=2)
    for r, (h, pos) in enumerate(rows):
        assert np.allclose(out[r], v[h // 2, : pos + 1].mean(axis=0), rtol=0, atol=1e-14)


def test_window_rows_equal_the_scoring_oracles_outputs():
    q, k, v = _case(7, n=24)
    n, w, G = 24, 5, 2
    for g in range(2):
        st = oracle.head_row_stats(q[:, n - w:, :], k, v, g, G, n, w)
        rows = [(g * G + t, n - w + i) for t in range(G) for i in range(w)]
        out = oracle.prefill_outputs(q, k, v, rows, Hq=4, Hkv=2)
        assert np.allclose(out, st["a"], rtol=1e-12, atol=1e-14)
