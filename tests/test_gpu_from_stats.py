"""Scoring from given window-row statistics (dropkv_score_from_stats), no pass 1.

The statistics come from dropkv_row_stats (what a prefill attention kernel
would hand over) and, separately, from the fp64 oracle; both runs must match
the oracle's scores to the bf16 tolerance and dropkv_score's outputs closely,
including heads with flagged rows (largest probability above 1/2), the
||v||^2 computed inside pass 2, and the row-group split of wide GQA groups.
"""

import math

import numpy as np
import pytest

import oracle
import kv_cache_eviction_pass1_amd as K
from kv_cache_eviction_pass1_amd import synth
from parity import RTOL, check_evictions, max_rel_err, run_oracle, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    yield


def _oracle_stats(case):
    qf, kf, vf = (oracle.as_f64(t, case.dtype) for t in (case.q, case.k, case.v))
    G = case.group
    m, rest, arg, a = [], [], [], []
    for g in range(case.Hkv):
        st = oracle.head_row_stats(qf, kf, vf, g, G, case.n, case.window)
        m.append(st["m"]); rest.append(st["rest"]); arg.append(st["jstar"]); a.append(st["a"])
    cat = lambda xs, dt: torch.from_numpy(np.concatenate(xs).astype(dt)).cuda().contiguous()
    return cat(m, np.float32), cat(rest, np.float32), cat(arg, np.int32), cat(a, np.float32)


def _compare(case, pool, ne, label):
    print(f"[from_stats] {label} Hq={case.Hq} Hkv={case.Hkv} n={case.n} w={case.window} evict={ne}", flush=True)
    q, k, v = to_torch(case)
    ref = run_oracle(case, pool, ne)
    base_sc, base_idx = K.score(q, k, v, pool_kernel=pool, n_evict=ne)
    base_sc = base_sc.cpu().numpy()
    for src in ("row_stats", "oracle"):
        if src == "row_stats":
            m, rest, arg, a = K.row_stats(q, k, v)
        else:
            m, rest, arg, a = _oracle_stats(case)
        sc, idx = K.score_from_stats(q, k, v, m.contiguous(), rest.contiguous(), arg.contiguous(),
                                     a.contiguous(), pool_kernel=pool, n_evict=ne)
        sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
        assert max_rel_err(sc, ref["P"]) <= RTOL["bf16"], src
        assert max_rel_err(sc, base_sc) <= 5e-3, src
        exact, jac = check_evictions(sc, idx, ref["P"], ref["S"], ref["evict"], ne, RTOL["bf16"])
        assert min(jac) > 0.99, src


@pytest.mark.parametrize("n,w,Hq,Hkv", [(2048, 32, 32, 8), (4161, 17, 6, 2), (1000, 3, 12, 3), (129, 64, 8, 1)])
def test_from_stats_matches(n, w, Hq, Hkv):
    case = synth.make_gaussian_case(Hq, Hkv, 128, n, w, dtype="bf16", seeds=(n, w, 7), sink=True, needles=8)
    _compare(case, 7, (n - w) // 2, "shapes")


def test_from_stats_pooled_tile_schedule():
    """Scoring from statistics on a shape that takes pass 2's pooled schedule
    (counters cleared by the init launch of this path)."""
    case = synth.make_gaussian_case(32, 8, 128, 8229, 32, dtype="bf16", seeds=(8, 2, 29), sink=True, needles=16)
    _compare(case, 7, 8229 - 411, "pooled schedule")


def test_from_stats_row_groups():
    case = synth.make_gaussian_case(28, 4, 128, 3000, 64, dtype="bf16", seeds=(1, 2, 3), sink=True, needles=16)
    _compare(case, 7, 2500, "qwen row groups")


def test_from_stats_flagged_rows():
    """Rows with p_max > 1/2 take the exact argmax fix-up here as well."""
    d, n, w, G = 128, 3000, 4, 2
    rng = np.random.default_rng(11)
    gaps = [0.0, 2.0, 7.0, 8.0, 10.0, 13.0, 16.0, 20.0]
    q = np.zeros((G, w, d), np.float32)
    k = (rng.standard_normal((1, n, d)) * 0.05).astype(np.float32)
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    for r in range(G * w):
        t, i = divmod(r, w)
        q[t, i, r] = 1.0
        k[0, 10 + 7 * r, r] = gaps[r] * math.sqrt(d)
    to_bf = synth.bf16_round_bits
    case = synth.Case(q=to_bf(q), k=to_bf(k), v=to_bf(v), n=n, window=w, Hq=G, Hkv=1, d=d, dtype="bf16")
    _compare(case, 3, 1500, "flagged")


def test_from_stats_rejects_bad_statistics():
    case = synth.make_gaussian_case(8, 2, 128, 500, 8, dtype="bf16", seeds=(1, 2, 3))
    q, k, v = to_torch(case)
    m, rest, arg, a = K.row_stats(q, k, v)
    m = m.clone()
    m[3] = float("nan")
    with pytest.raises(K.DropKVNonFiniteError):
        K.score_from_stats(q, k, v, m, rest.contiguous(), arg.contiguous(), a.contiguous(),
                           pool_kernel=3, n_evict=100)
    with pytest.raises(K.DropKVInvalidError):  # fp32 inputs are not on this path
        qf, kf, vf = (t.float() for t in (q, k, v))
        K.score_from_stats(qf, kf, vf, m, rest, arg, a, pool_kernel=3, n_evict=100)


def test_from_stats_async_matches_sync():
    case = synth.make_gaussian_case(32, 8, 128, 5000, 64, dtype="bf16", seeds=(4, 4, 4), sink=True, needles=8)
    q, k, v = to_torch(case)
    m, rest, arg, a = (t.contiguous() for t in K.row_stats(q, k, v))
    print("[from_stats] async vs sync", flush=True)
    sc0, ix0 = K.score_from_stats(q, k, v, m, rest, arg, a, pool_kernel=7, n_evict=4000)
    ws = torch.empty(K.workspace_bytes(K.BF16, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device="cuda")
    st = torch.full((1,), 123, dtype=torch.int32, device="cuda")  # the call clears it
    for _ in range(2):
        sc1, ix1 = K.score_from_stats(q, k, v, m, rest, arg, a, pool_kernel=7, n_evict=4000,
                                      workspace=ws, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(sc0, sc1) and torch.equal(ix0, ix1)
