"""Delete-and-recompute reference for DropKV scores (tiny inputs only).

Independent of the oracle: for every window query and every visible token j
it literally removes j, re-normalises the softmax over the remaining visible
keys, recomputes the attention output and takes the squared norm of the
change. The DropKV write-up reports the same kind of check for its own
implementation (section 结果与独立对照, where each token is really removed and
the softmax recomputed), and section 核心公式 defines Delta_j as the closed
form of exactly this single-token removal.

Pure Python loops over rows and tokens; numpy only for small vectors.
"""

from __future__ import annotations

import math

import numpy as np


def _softmax_output(logits, values, keep):
    """Output of softmax attention restricted to the index list `keep`."""
    top = max(logits[j] for j in keep)
    weights = [math.exp(logits[j] - top) for j in keep]
    total = math.fsum(weights)
    out = np.zeros(values.shape[1])
    for wgt, j in zip(weights, keep):
        out += (wgt / total) * values[j]
    return out


def brute_force_scores(q, k, v, n, window, Hq, Hkv):
    """s[h][j]: sum over window rows of h of ||a^(-j) - a||^2; S[g][j] = mean over the group.

    q [Hq][w][d], k/v [Hkv][n][d] as float64. Row i of the window is at
    position n - window + i and sees keys 0..n-window+i.
    """
    G = Hq // Hkv
    d = q.shape[2]
    s = np.zeros((Hq, n))
    for h in range(Hq):
        g = h // G
        for i in range(window):
            pos = n - window + i
            visible = list(range(pos + 1))
            logits = [float(np.dot(q[h, i], k[g, j])) / math.sqrt(d) for j in range(n)]
            full = _softmax_output(logits, v[g], visible)
            for j in visible:
                rest = [t for t in visible if t != j]
                reduced = _softmax_output(logits, v[g], rest)
                delta = reduced - full
                s[h, j] += float(np.dot(delta, delta))
    S = s.reshape(Hkv, G, n).mean(axis=1)
    return s, S


def brute_force_joint(q, k, v, g, G, n, window, E):
    """J_g(E) by literal deletion: the output change of removing the whole set E.

    For every query head h of KV head g and every window row i (position
    n - window + i, keys 0..position visible), the softmax output over the
    visible keys and over the visible keys outside E are recomputed from the
    logits, and the squared norm of their difference is summed; the sum is
    divided by G (the GQA mean). Pure Python loops, like brute_force_scores.
    """
    d = q.shape[2]
    removed = set(int(j) for j in E)
    total = 0.0
    for t in range(G):
        h = g * G + t
        for i in range(window):
            pos = n - window + i
            visible = list(range(pos + 1))
            logits = [float(np.dot(q[h, i], k[g, j])) / math.sqrt(d) for j in range(n)]
            full = _softmax_output(logits, v[g], visible)
            rest = [j for j in visible if j not in removed]
            reduced = _softmax_output(logits, v[g], rest)
            delta = reduced - full
            total += float(np.dot(delta, delta))
    return total / G
