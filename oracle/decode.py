"""Decode-time rescoring with a sliding observation window (CPU, fp64).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only tests, the
smoke check and the benchmark's CPU leg use it; the HIP library never does.

Pages: the atlas summary (Limitations) names a decode-time kernel as future
work and calls per-step decode bandwidth-bound; the write-up's core formula
(核心公式) defines the score as a sum over the observation-window queries of
||Delta_j||^2, averaged over the query heads of a KV head. The pages say no
more about decode. The reading here is the plainest one that keeps that
definition while tokens are appended:

  * the observation window is always the last w query positions of the
    current cache (causal tail alignment, as at prefill);
  * one decode step appends one token (its key and value at position n, and
    the query rows of all Hq heads at that position): the window gains the row
    at the new position and loses its oldest row, at position n - w;
  * a window row's attention and its ||Delta_j||^2 depend only on the keys it
    sees (0 .. its position), which appending does not change, so the raw
    score of the grown cache is the old one plus the new row's terms minus
    the leaving row's terms, with the new token's entry starting from the new
    row's term alone;
  * re-eviction (max-pool, protect the window, evict the smallest) runs on the
    maintained raw score exactly as at prefill; after an eviction every row's
    softmax changes, so scoring starts again from the compacted cache.

decode_step follows those steps literally; decode_scratch recomputes the same
score from the definition (head_scores on the final cache), which is what the
pins compare against.
"""

from __future__ import annotations

from typing import Dict

import numpy as np

from .dropkv_oracle import (SINGULAR_REST_MASS, SingularRow, as_f64, head_scores, maxpool1d_same,
                            perturbation_sq, protect_window, evict_smallest, row_attention)


def decode_scratch(q_win, k, v, *, n: int, window: int, Hq: int, Hkv: int, d: int,
                   dtype: str = "f64") -> np.ndarray:
    """Raw GQA-mean scores S [Hkv][n] of the first n cache tokens with the
    window queries q_win [Hq][window][d] (positions n - window .. n - 1)."""
    G = Hq // Hkv
    qf = as_f64(q_win, dtype)
    kf = as_f64(k, dtype)[:, :n]
    vf = as_f64(v, dtype)[:, :n]
    return np.stack([head_scores(qf, kf, vf, g, G, n, window)["S"] for g in range(Hkv)])


def decode_init(q_win, k, v, *, n: int, window: int, Hq: int, Hkv: int, d: int,
                dtype: str = "f64") -> Dict[str, object]:
    """State after scoring an n-token cache: the raw score S and the window's
    query rows (oldest first)."""
    S = decode_scratch(q_win, k, v, n=n, window=window, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype)
    return {"S": S, "q_win": as_f64(q_win, dtype).copy(), "n": n, "window": window,
            "Hq": Hq, "Hkv": Hkv, "d": d}


def _row_terms(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, pos: int, head: int,
               i: int) -> np.ndarray:
    """||Delta_j||^2 of query rows qrows [G][d], all at position pos, for every
    token j < len(K) (zero beyond pos). Rejects a singular row."""
    G = qrows.shape[0]
    st = row_attention(qrows, K, np.full(G, pos, dtype=np.int64))
    bad = np.nonzero(st["rest"] <= SINGULAR_REST_MASS)[0]
    if bad.size:
        r = int(bad[0])
        raise SingularRow(head + r, i, int(st["jstar"][r]), float(st["rest"][r]))
    st["a"] = (st["e"] / st["L"][:, None]) @ V
    return perturbation_sq(st, V)


def decode_step(state: Dict[str, object], q_new, k, v, dtype: str = "f64") -> Dict[str, object]:
    """One appended token: k, v hold at least n + 1 tokens per KV head (the new
    one at index n), q_new [Hq][d] is the new position's query rows."""
    n, w = int(state["n"]), int(state["window"])
    Hq, Hkv = int(state["Hq"]), int(state["Hkv"])
    G = Hq // Hkv
    n1 = n + 1
    kf = as_f64(k, dtype)[:, :n1]
    vf = as_f64(v, dtype)[:, :n1]
    qn = as_f64(q_new, dtype).reshape(Hq, -1)
    q_win = state["q_win"]
    S_old = state["S"]
    S = np.zeros((Hkv, n1))
    S[:, :n] = S_old
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        add = _row_terms(qn[heads], kf[g], vf[g], n1 - 1, g * G, w - 1)
        sub = _row_terms(q_win[heads, 0], kf[g], vf[g], n1 - 1 - w, g * G, 0)
        S[g] += (add.sum(axis=0) - sub.sum(axis=0)) / G
    q_next = np.concatenate([q_win[:, 1:], qn[:, None, :]], axis=1)
    out = dict(state)
    out.update({"S": S, "q_win": q_next, "n": n1})
    return out


def decode_select(state: Dict[str, object], pool_kernel: int, n_evict: int) -> Dict[str, np.ndarray]:
    """Re-eviction on the maintained score: pool, protect the window, evict the smallest."""
    P = protect_window(maxpool1d_same(state["S"], pool_kernel), int(state["window"]))
    return {"P": P, "evict": evict_smallest(P, n_evict)}
