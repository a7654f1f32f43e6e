"""Approximation-ratio diagnostic of the DropKV selection (CPU, fp64).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only tests and the
benchmark's CPU leg use it; the HIP library never does.

Pages: the paper's abstract (fugumt page) and the write-up's background
section (背景与主要改动) state that choosing the evicted set jointly, to
minimise the output change of removing the whole set, is NP-hard, and that
DropKV decouples it into independent single-token scores; the paper reports
an empirical approximation ratio of that decoupling (atlas summary, Key
results). The joint objective is not printed on the pages; the reading used
here is the plainest one consistent with the single-token score:

    J_g(E) = (1/G) * sum over the query heads h of KV head g
                     sum over the window rows t of ||a_t^(-E) - a_t||^2,

where a_t^(-E) is the attention output of row t with the tokens of E removed
and the softmax renormalised over the remaining visible tokens. For E = {j}
this is exactly the pre-pooling score S_g(j) (the tests pin that), so the
DropKV choice is the bottom-k of J over single tokens (with pooling on top),
and the ratio J_g(E_DropKV) / min_{|E| = k} J_g(E) measures what the
decoupling gives up. E ranges over the tokens outside the protected window.
"""

from __future__ import annotations

import itertools
import math
from typing import Dict, Iterable

import numpy as np

from .dropkv_oracle import (as_f64, evict_smallest, group_rows, head_scores, maxpool1d_same,
                            protect_window, window_positions)


def _logits(qf, kf, g: int, G: int, n: int, w: int) -> np.ndarray:
    """Logits of KV head g's window rows (row r = t*w + i), -inf where not visible."""
    d = kf.shape[2]
    x = group_rows(qf, g, G) @ kf[g].T / math.sqrt(d)
    pos = np.tile(window_positions(n, w), G)
    return np.where(np.arange(n)[None, :] <= pos[:, None], x, -np.inf)


def _outputs(x: np.ndarray, V: np.ndarray) -> np.ndarray:
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return (e / e.sum(axis=1, keepdims=True)) @ V


def joint_objective(q, k, v, g: int, G: int, n: int, w: int, E: Iterable[int],
                    dtype: str = "f64") -> float:
    """J_g(E): the output change of removing the token set E from KV head g (see module doc)."""
    qf, kf, vf = as_f64(q, dtype), as_f64(k, dtype), as_f64(v, dtype)
    x = _logits(qf, kf, g, G, n, w)
    a = _outputs(x, vf[g])
    E = np.asarray(list(E), dtype=np.int64)
    if E.size == 0:
        return 0.0
    xr = x.copy()
    xr[:, E] = -np.inf
    ar = _outputs(xr, vf[g])
    return float(np.sum((ar - a) ** 2) / G)


def approx_ratio(q, k, v, *, n: int, window: int, Hq: int, Hkv: int, d: int, n_evict: int,
                 pool_kernel: int, dtype: str = "f64") -> Dict[str, np.ndarray]:
    """Per KV head: J of the DropKV set (pooled scores), of the unpooled bottom-k,
    and the exact minimum over all size-n_evict subsets of the unprotected tokens
    (brute force: use tiny n only)."""
    G = Hq // Hkv
    qf, kf, vf = as_f64(q, dtype), as_f64(k, dtype), as_f64(v, dtype)
    cand = np.arange(n - window)
    out = {"J_dropkv": np.zeros(Hkv), "J_unpooled": np.zeros(Hkv), "J_opt": np.zeros(Hkv),
           "E_opt": []}
    for g in range(Hkv):
        S = head_scores(qf, kf, vf, g, G, n, window)["S"]
        P = protect_window(maxpool1d_same(S[None, :], pool_kernel), window)
        E_d = evict_smallest(P, n_evict)[0]
        E_u = evict_smallest(protect_window(S[None, :], window), n_evict)[0]
        x = _logits(qf, kf, g, G, n, window)
        a = _outputs(x, vf[g])
        best, best_E = np.inf, None
        for E in itertools.combinations(cand, n_evict):
            xr = x.copy()
            xr[:, list(E)] = -np.inf
            J = float(np.sum((_outputs(xr, vf[g]) - a) ** 2) / G)
            if J < best:
                best, best_E = J, E
        out["J_dropkv"][g] = joint_objective(qf, kf, vf, g, G, n, window, E_d)
        out["J_unpooled"][g] = joint_objective(qf, kf, vf, g, G, n, window, E_u)
        out["J_opt"][g] = best
        out["E_opt"].append(np.asarray(best_E, dtype=np.int64))
    out["ratio"] = out["J_dropkv"] / out["J_opt"]
    out["ratio_unpooled"] = out["J_unpooled"] / out["J_opt"]
    return out
