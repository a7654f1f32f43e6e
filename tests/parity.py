"""Helpers that compare the HIP library's outputs with the fp64 oracle.

Tolerances: relative 2e-2 on scores for bf16 inputs and 1e-5 for fp32
inputs, on every finite entry; +inf entries (the protected window) must match
exactly. Evicted sets must always be the bottom-n_evict of the GPU's own
pooled scores under (score, index); they must equal the oracle's set exactly
when the oracle's k-th / (k+1)-th gap exceeds twice the tolerance, or when no
oracle score other than the boundary value lies within twice the tolerance of
it; otherwise every index in which the two sets differ must have an oracle
score within the band that the measured score error allows around the
boundary value (check_evictions).
"""

from __future__ import annotations

import numpy as np

import oracle

RTOL = {"bf16": 2e-2, "f32": 1e-5}


def to_torch(case, device="cuda"):
    import torch
    if case.dtype == "bf16":
        conv = lambda a: torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return tuple(conv(t).to(device).contiguous() for t in (case.q, case.k, case.v))


def run_oracle(case, pool_kernel, n_evict, heads=None):
    return oracle.dropkv_oracle(case.q, case.k, case.v, n=case.n, window=case.window, Hq=case.Hq,
                                Hkv=case.Hkv, d=case.d, pool_kernel=pool_kernel, n_evict=n_evict,
                                dtype=case.dtype, heads=heads)


def max_rel_err(gpu, ref, floor_rel=1e-30):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_ref = np.isinf(ref)
    assert np.array_equal(np.isinf(gpu), inf_ref), "+inf positions differ"
    assert np.all(gpu[inf_ref] > 0), "-inf in GPU scores"
    fin = ~inf_ref
    if not fin.any():
        return 0.0
    assert np.all(np.isfinite(gpu[fin])), "non-finite GPU score"
    scale = np.max(np.abs(ref[fin]))
    floor = max(floor_rel * scale, 1e-300)
    err = np.abs(gpu[fin] - ref[fin]) / np.maximum(np.abs(ref[fin]), floor)
    return float(err.max())


def own_bottom_k(scores_row, k):
    return np.sort(np.argsort(scores_row, kind="stable")[:k])


def symdiff_band(e):
    """Relative band around the oracle's boundary value tau that every index
    of the symmetric difference must fall in, when every GPU pooled score is
    within relative e of the oracle's.

    If |g_j - r_j| <= e r_j for all j, the k-th smallest GPU value lies in
    [(1-e) tau, (1+e) tau]; an index the GPU evicts and the oracle keeps has
    r_j >= tau and g_j <= (1+e) tau, so r_j <= tau (1+e)/(1-e); one the oracle
    evicts and the GPU keeps has r_j <= tau and r_j >= tau (1-e)/(1+e).
    """
    return (1.0 - e) / (1.0 + e), (1.0 + e) / (1.0 - e)


def check_evictions(gpu_scores, gpu_idx, ref_P, ref_S, ref_idx, n_evict, rtol, report=None):
    """Returns (n_exact_checked, jaccards). Asserts, per KV head:

    (a) the GPU set is the bottom-n_evict of the GPU's own pooled scores
        under (score, index), strictly ascending;
    (b) gap rule: when the oracle's sorted pooled scores satisfy
        P_(k+1) - P_(k) > 2 rtol P_(k), the GPU set equals the oracle's;
    (c) plateau rule: when no oracle value other than tau = P_(k) (raw or
        pooled) lies within 2 rtol of tau, the GPU set equals the oracle's
        (pooling plateaus copy tau bit for bit on both sides);
    (d) always: every index in the symmetric difference has an oracle pooled
        score inside symdiff_band(e) around tau, e being this head's
        measured largest relative error of the pooled scores (e <= rtol, so
        the band lies inside tau (1 +- 2 rtol) to first order), and the two
        one-sided differences have equal size.
    `report` (a dict) counts heads per rule: gap, plateau, band, sizes of
    the symmetric differences.
    """
    gpu_scores = np.asarray(gpu_scores)
    gpu_idx = np.asarray(gpu_idx)
    exact, jac = 0, []
    rep = report if report is not None else {}
    for key in ("heads", "gap_exact", "plateau_exact", "band_checked", "symdiff_max", "band_used_max"):
        rep.setdefault(key, 0)
    for g in range(gpu_scores.shape[0]):
        rep["heads"] += 1
        if n_evict == 0:
            assert gpu_idx.shape[1] == 0
            continue
        own = own_bottom_k(gpu_scores[g], n_evict)
        assert np.array_equal(gpu_idx[g], own), f"head {g}: not the bottom-k of its own scores"
        assert np.all(np.diff(gpu_idx[g]) > 0), "indices not strictly ascending"
        ref = ref_idx[g]
        inter = np.intersect1d(ref, gpu_idx[g]).size
        jac.append(inter / max(1, np.union1d(ref, gpu_idx[g]).size))
        srt = np.sort(ref_P[g])
        tau = srt[n_evict - 1]
        nxt = srt[n_evict] if n_evict < srt.size else np.inf
        # (b) the k-th / (k+1)-th gap rule
        if nxt - tau > 2 * rtol * tau:
            assert np.array_equal(gpu_idx[g], ref), f"head {g}: evicted set differs (gap rule)"
            rep["gap_exact"] += 1
            exact += 1
            continue
        # (c) no other oracle value near tau
        band = 2 * rtol * abs(tau)
        near_P = np.abs(ref_P[g] - tau) <= band
        near_S = np.abs(ref_S[g] - tau) <= band
        ambiguous = np.any(near_P & (ref_P[g] != tau)) or np.any(near_S & (ref_S[g] != tau))
        if not ambiguous:
            assert np.array_equal(gpu_idx[g], ref), f"head {g}: evicted set differs (plateau rule)"
            rep["plateau_exact"] += 1
            exact += 1
            continue
        # (d) every difference lies where the measured score error allows
        e = max_rel_err(gpu_scores[g], ref_P[g])
        assert e <= rtol, f"head {g}: pooled scores rel err {e:.3e}"
        lo, hi = symdiff_band(e)
        only_gpu = np.setdiff1d(gpu_idx[g], ref)
        only_ref = np.setdiff1d(ref, gpu_idx[g])
        assert only_gpu.size == only_ref.size, f"head {g}: one-sided differences of unequal size"
        diff = np.concatenate([only_gpu, only_ref])
        if diff.size:
            rv = ref_P[g][diff]
            slack = 1e-12 * tau
            bad = (rv < tau * lo - slack) | (rv > tau * hi + slack)
            assert not np.any(bad), (
                f"head {g}: {int(bad.sum())} differing indices outside the error band "
                f"[{tau * lo:.6e}, {tau * hi:.6e}] (e = {e:.3e}), e.g. index {int(diff[bad][0])} "
                f"with oracle score {float(rv[bad][0]):.6e}")
            used = float(np.max(np.abs(rv / tau - 1.0)))
            rep["band_used_max"] = max(rep["band_used_max"], used)
        rep["band_checked"] += 1
        rep["symdiff_max"] = max(rep["symdiff_max"], int(only_gpu.size))
    return exact, jac


def sample_tokens(case, g, rng, n_random=96, chunk=4096):
    n, w = case.n, case.window
    picks = [0, 1, 2, n - w - 1, n - w, n - w + 1, n - 2, n - 1]
    picks += [c for b in range(chunk, n, chunk) for c in (b - 1, b)]
    if case.needle_pos is not None:
        picks += [int(p) for p in case.needle_pos[g]]
    picks += [int(t) for t in rng.choice(n, size=n_random, replace=False)]
    return np.unique(np.clip(np.asarray(picks), 0, n - 1))


def check_sampled(case, g, pool, S_gpu, P_gpu, rng):
    """Raw and pooled scores of head g on sampled tokens, against the oracle."""
    G, n, w = case.group, case.n, case.window
    half = pool // 2
    toks = sample_tokens(case, g, rng)
    need = np.unique(np.clip((toks[:, None] + np.arange(-half, half + 1)[None, :]).ravel(), 0, n - 1))
    q = oracle.as_f64(case.q, case.dtype)
    k = oracle.as_f64(case.k, case.dtype)
    v = oracle.as_f64(case.v, case.dtype)
    hs = oracle.head_scores(q, k, v, g, G, n, w, tokens=need)
    S_ref = dict(zip(need.tolist(), hs["S"].tolist()))
    ref_S = np.array([S_ref[int(t)] for t in toks])
    ref_P = np.array([max(S_ref[int(u)] for u in range(max(0, t - half), min(n, t + half + 1)))
                      for t in toks])
    ref_P = np.where(toks >= n - w, np.inf, ref_P)
    rtol = RTOL[case.dtype]
    e_S = max_rel_err(S_gpu[g, toks], ref_S)
    e_P = max_rel_err(P_gpu[g, toks], ref_P)
    assert e_S <= rtol, f"head {g}: sampled raw scores rel err {e_S:.3e}"
    assert e_P <= rtol, f"head {g}: sampled pooled scores rel err {e_P:.3e}"
    return e_S, e_P
