"""fp64 CPU oracle for DropKV eviction scoring.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code, constant or helper with the HIP library.

What it computes, written from the DropKV pages (arXiv 2610.22130):

* Write-up "DropKV：精确单项输出扰动评分组件" (daiwk.github.io), section
  核心公式 (core formula), displayed equation: with p = softmax(Kq/sqrt(d)) and
  a = sum_j p_j v_j, removing token j alone changes the output by
  Delta_j = p_j/(1-p_j) (a - v_j), and the token's score is
  s_j = sum over the observation-window queries t of ||Delta_j^(t)||_2^2.
* Same section, the prose after the equation: Algorithm 1 max-pools the
  scores (MaxPool1D), sets the last observation window's scores to +inf and
  evicts the smallest; under GQA the scores of the query heads that share one
  physical KV head are averaged; a probability that rounds to 1 makes exact
  single-token removal singular and the input is rejected (no epsilon).
* Same write-up, section 代码映射与边界 (code map): causal tail alignment
  (the window queries are the last positions of the sequence) and the
  per-physical-KV-head scores and evict indices it returns.
* The pipeline figure of section 背景与主要改动: window attention -> squared
  single-token perturbation -> accumulate over queries and merge heads ->
  max pooling and recent protection -> evict the smallest (so the GQA mean
  comes before pooling).

Readings where the pages are silent (all listed in the design notes):
  - query row i of the window sits at position n-w+i and sees keys 0..n-w+i;
  - query head h belongs to KV head h // G (contiguous groups, G = Hq/Hkv);
  - MaxPool1D: odd kernel k, stride 1, "same" padding (window clipped to
    [0, n)), over the full length n, then protection of the last w positions;
  - "rounds to 1" is taken in binary32: a row is singular iff
    R = sum_{j != j*} exp(x_j - x_{j*}) <= 2**-24 (then 1/(1+R) == 1.0f);
  - eviction order is (score, index): among equal scores the lower index is
    evicted first; indices are returned ascending;
  - argmax ties go to the lowest index.

Everything is float64. bf16 inputs enter as their exact values.
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

# binary32 "rounds to 1" threshold for the singular-input rule.
SINGULAR_REST_MASS = 2.0 ** -24


class SingularRow(ValueError):
    """A window row whose largest probability rounds to 1 (rejected)."""

    def __init__(self, head: int, row: int, jstar: int, rest_mass: float):
        super().__init__(f"singular row: query head {head}, window row {row}, "
                         f"argmax token {jstar}, rest mass {rest_mass:.3e}")
        self.head, self.row, self.jstar, self.rest_mass = head, row, jstar, rest_mass


class NonFiniteInput(ValueError):
    """An input holds NaN or inf."""


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the top 16 bits of a binary32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def window_positions(n: int, w: int) -> np.ndarray:
    """Causal tail alignment: window row i is at sequence position n-w+i."""
    return np.arange(n - w, n, dtype=np.int64)


def group_rows(q: np.ndarray, g: int, G: int) -> np.ndarray:
    """Queries of the heads gG..gG+G-1 stacked head-major: row r = t*w + i."""
    Hq, w, d = q.shape
    return q[g * G:(g + 1) * G].reshape(G * w, d)


def row_attention(qrows: np.ndarray, K: np.ndarray, pos: np.ndarray) -> Dict[str, np.ndarray]:
    """Causal softmax attention statistics of query rows against keys K.

    qrows: [R][d]; K: [n][d]; pos[r] = the row's position (keys 0..pos[r]
    visible). Returns per row: x (logits [R][n], -inf where not visible),
    jstar, m = x[jstar], e = exp(x - m), rest = sum_{j != jstar} e_j (summed
    directly, never as L - 1) and L = 1 + rest, so p = e / L.
    Core formula: p = softmax(Kq / sqrt(d)).
    """
    d = K.shape[1]
    x = (qrows @ K.T) / math.sqrt(d)
    cols = np.arange(K.shape[0])
    visible = cols[None, :] <= pos[:, None]
    x = np.where(visible, x, -np.inf)
    jstar = np.argmax(x, axis=1)  # first (lowest-index) maximum
    rr = np.arange(x.shape[0])
    m = x[rr, jstar]
    e = np.exp(x - m[:, None])  # exp(-inf) = 0 for masked keys
    e_rest = e.copy()
    e_rest[rr, jstar] = 0.0
    rest = e_rest.sum(axis=1)
    L = 1.0 + rest
    return {"x": x, "jstar": jstar, "m": m, "e": e, "rest": rest, "L": L}


def head_row_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: int, G: int,
                   n: int, w: int, check_singular: bool = True) -> Dict[str, np.ndarray]:
    """Per window row of KV head g: attention stats and the output a = sum p_j v_j."""
    qrows = group_rows(q, g, G)
    pos = np.tile(window_positions(n, w), G)
    st = row_attention(qrows, k[g], pos)
    if check_singular:
        bad = np.nonzero(st["rest"] <= SINGULAR_REST_MASS)[0]
        if bad.size:
            r = int(bad[0])
            raise SingularRow(g * G + r // w, r % w, int(st["jstar"][r]), float(st["rest"][r]))
    p = st["e"] / st["L"][:, None]
    st["p"] = p
    st["a"] = p @ v[g]
    st["pos"] = pos
    return st


def perturbation_sq(st: Dict[str, np.ndarray], V: np.ndarray,
                    tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """||Delta_j^(t)||^2 for every window row t (rows) and token j (columns).

    Delta_j = p_j / (1 - p_j) * (a - v_j)  (core formula). 1 - p_j is formed as
    (L - e_j) / L, and as rest / L for the argmax token, so no cancellation
    against 1 occurs. ||a - v_j||^2 is the direct sum of squared differences.
    Tokens a row cannot see have p_j = 0 and contribute 0.
    """
    if tokens is None:
        tokens = np.arange(V.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    e = st["e"][:, tokens]
    L = st["L"][:, None]
    p = e / L
    one_minus_p = (L - e) / L
    is_star = tokens[None, :] == st["jstar"][:, None]
    one_minus_p = np.where(is_star, (st["rest"] / st["L"])[:, None], one_minus_p)
    ratio = p / one_minus_p
    a = st["a"]
    Vt = V[tokens]
    dist2 = np.empty((a.shape[0], tokens.size))
    for r in range(a.shape[0]):
        diff = a[r][None, :] - Vt
        dist2[r] = np.sum(diff * diff, axis=1)
    return ratio * ratio * dist2


def head_scores(q, k, v, g: int, G: int, n: int, w: int,
                tokens: Optional[np.ndarray] = None, stats=None) -> Dict[str, np.ndarray]:
    """Scores of KV head g.

    per_head[t][j] = s_j for query head gG+t: the sum over its window rows
    of ||Delta_j||^2 (core formula's sum over the observation window);
    S[j] = mean over the G query heads (GQA rule: mean over the query heads
    of one physical KV head).
    """
    st = stats if stats is not None else head_row_stats(q, k, v, g, G, n, w)
    contrib = perturbation_sq(st, v[g], tokens)
    per_head = contrib.reshape(G, w, -1).sum(axis=1)
    S = per_head.sum(axis=0) / G
    return {"per_head": per_head, "S": S, "stats": st}


def maxpool1d_same(S: np.ndarray, kernel: int) -> np.ndarray:
    """MaxPool1D along the last axis: stride 1, odd kernel, window clipped to [0, n)."""
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and >= 1")
    n = S.shape[-1]
    half = kernel // 2
    out = np.empty_like(S)
    for j in range(n):
        lo, hi = max(0, j - half), min(n, j + half + 1)
        out[..., j] = S[..., lo:hi].max(axis=-1)
    return out


def protect_window(P: np.ndarray, w: int) -> np.ndarray:
    """Set the last observation window's scores to +inf (Algorithm 1, as described)."""
    out = P.copy()
    out[..., P.shape[-1] - w:] = np.inf
    return out


def evict_smallest(P: np.ndarray, n_evict: int) -> np.ndarray:
    """The n_evict smallest scores per row under the order (score, index), ascending indices."""
    P = np.atleast_2d(P)
    out = np.empty((P.shape[0], n_evict), dtype=np.int64)
    for g in range(P.shape[0]):
        order = np.argsort(P[g], kind="stable")[:n_evict]
        out[g] = np.sort(order)
    return out


def compact_cache(k: np.ndarray, v: np.ndarray, evict: np.ndarray):
    """Cache compaction, the step after scoring.

    Write-up section 代码映射与边界 (code map): the scorer hands back, per
    physical KV head, the indices of the tokens to drop, and the caller removes
    them from its cache. Per head g, the result holds the rows k[g, j], v[g, j]
    of every j that evict[g] does not list, in ascending j (the order of the
    cache). The rows are copied as they are (bit patterns included).
    Raises ValueError unless each evict[g] is strictly increasing inside [0, n).
    """
    evict = np.asarray(evict, dtype=np.int64).reshape(k.shape[0], -1)
    Hkv, n = k.shape[0], k.shape[1]
    if v.shape != k.shape:
        raise ValueError("k and v must have one shape")
    n_keep = n - evict.shape[1]
    ok = np.empty((Hkv, n_keep) + k.shape[2:], dtype=k.dtype)
    ov = np.empty((Hkv, n_keep) + v.shape[2:], dtype=v.dtype)
    for g in range(Hkv):
        e = evict[g]
        if e.size and (e[0] < 0 or e[-1] >= n or np.any(np.diff(e) <= 0)):
            raise ValueError("eviction list must be strictly increasing inside [0, n)")
        keep = np.ones(n, dtype=bool)
        keep[e] = False
        ok[g] = k[g][keep]
        ov[g] = v[g][keep]
    return ok, ov


def check_args(n: int, window: int, Hq: int, Hkv: int, d: int, pool_kernel: int, n_evict: int) -> None:
    w = window
    if not (1 <= w < n):
        raise ValueError("need 1 <= window < n")
    if Hq < 1 or Hkv < 1 or Hq % Hkv:
        raise ValueError("need Hq a positive multiple of Hkv")
    if d < 1:
        raise ValueError("need d >= 1")
    if pool_kernel < 1 or pool_kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and >= 1")
    if not (0 <= n_evict <= n - w):
        raise ValueError("need 0 <= n_evict <= n - window")


def dropkv_oracle(q, k, v, *, n: int, window: int, Hq: int, Hkv: int, d: int,
                  pool_kernel: int, n_evict: int, dtype: str = "f64",
                  heads: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """The full DropKV scoring of one sequence.

    q [Hq][w][d], k/v [Hkv][n][d] (dtype "bf16" bit patterns, "f32" or "f64").
    Returns raw per-query-head scores s, GQA-mean scores S, pooled + protected
    scores P and the evicted indices per KV head (all KV heads, or `heads`).
    Raises SingularRow / NonFiniteInput / ValueError.
    """
    check_args(n, window, Hq, Hkv, d, pool_kernel, n_evict)
    qf, kf, vf = as_f64(q, dtype), as_f64(k, dtype), as_f64(v, dtype)
    if qf.shape != (Hq, window, d) or kf.shape != (Hkv, n, d) or vf.shape != (Hkv, n, d):
        raise ValueError("shape mismatch")
    for t in (qf, kf, vf):
        if not np.all(np.isfinite(t)):
            raise NonFiniteInput("input holds NaN or inf")
    G = Hq // Hkv
    heads = list(range(Hkv)) if heads is None else list(heads)
    per_head = np.zeros((len(heads) * G, n))
    S = np.zeros((len(heads), n))
    stats = []
    for idx, g in enumerate(heads):
        res = head_scores(qf, kf, vf, g, G, n, window)
        per_head[idx * G:(idx + 1) * G] = res["per_head"]
        S[idx] = res["S"]
        stats.append(res["stats"])
    P = protect_window(maxpool1d_same(S, pool_kernel), window)
    evict = evict_smallest(P, n_evict)
    return {"s": per_head, "S": S, "P": P, "evict": evict, "stats": stats, "heads": heads}
