"""The MFMA path (bf16, d = 128) against the fp64 oracle, through the C ABI.

Covers the pass-1 statistics export, tile/chunk boundaries, rows that are not
a multiple of the 32-row MFMA block, the row-group split of wide GQA groups,
and rows whose largest probability exceeds 1/2 (handled by the exact argmax
fix-up), down to rest masses near the singular threshold.
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
    assert K.uses_mfma(K.BF16, 128), "bf16 d=128 must take the MFMA path"
    yield


def _compare(case, pool, ne, label=""):
    print(f"[mfma] {label} Hq={case.Hq} Hkv={case.Hkv} n={case.n} w={case.window} pool={pool} evict={ne}",
          flush=True)
    q, k, v = to_torch(case)
    scores, idx = K.score(q, k, v, pool_kernel=pool, n_evict=ne)
    S = K.raw_scores(q, k, v)
    scores, idx, S = scores.cpu().numpy(), idx.cpu().numpy(), S.cpu().numpy()
    ref = run_oracle(case, pool, ne)
    rtol = RTOL["bf16"]
    e_S = max_rel_err(S, ref["S"])
    e_P = max_rel_err(scores, ref["P"])
    assert e_S <= rtol, f"raw S rel err {e_S:.3e}"
    assert e_P <= rtol, f"pooled rel err {e_P:.3e}"
    exact, jac = check_evictions(scores, idx, ref["P"], ref["S"], ref["evict"], ne, rtol)
    return e_S, exact, jac


@pytest.mark.parametrize("n,w,Hq,Hkv", [
    (65, 1, 4, 2), (127, 63, 4, 4), (129, 64, 8, 1), (200, 65, 2, 1), (3, 2, 4, 2),
    (1000, 3, 12, 3), (2048, 32, 32, 8), (4161, 17, 6, 2),
])
def test_mfma_tile_and_row_boundaries(n, w, Hq, Hkv):
    case = synth.make_gaussian_case(Hq, Hkv, 128, n, w, dtype="bf16", seeds=(n, w, Hq),
                                    sink=n > w + 2, needles=min(8, max(0, n - w - 2)))
    ne = (n - w) // 2
    _compare(case, 7 if n > 16 else 3, ne, "bounds")


@pytest.mark.parametrize("n,w,Hq,Hkv", [(8229, 32, 32, 8), (8292, 64, 28, 4), (65600, 32, 8, 1)])
def test_mfma_pooled_tile_schedule(n, w, Hq, Hkv):
    """Shapes long enough for pass 2's pooled schedule (static shares of three
    quarters of the tiles, the rest claimed one tile at a time): a ragged last
    tile and the masked window tiles sit in the pool; two row groups with
    their own counters; one KV head over 256 workgroups."""
    case = synth.make_gaussian_case(Hq, Hkv, 128, n, w, dtype="bf16", seeds=(n, w, Hq), sink=True, needles=16)
    _compare(case, 7, n - n // 20, "pooled schedule")


def test_mfma_row_groups_qwen_shape():
    """28 query heads over 4 KV heads with w = 64: 448 rows per KV head, two row groups."""
    case = synth.make_gaussian_case(28, 4, 128, 3000, 64, dtype="bf16", seeds=(42, 43, 44),
                                    sink=True, needles=16)
    _compare(case, 7, 2500, "qwen-rowgroups")


def test_mfma_row_stats_export():
    case = synth.make_gaussian_case(8, 2, 128, 3000, 16, dtype="bf16", seeds=(4, 5, 6), sink=True, needles=8)
    q, k, v = to_torch(case)
    m, rest, arg, a = (t.cpu().numpy() for t in K.row_stats(q, k, v))
    qf, kf, vf = (oracle.as_f64(t, "bf16") for t in (case.q, case.k, case.v))
    G = case.group
    for g in range(case.Hkv):
        st = oracle.head_row_stats(qf, kf, vf, g, G, case.n, case.window)
        rows = slice(g * G * case.window, (g + 1) * G * case.window)
        assert np.allclose(m[rows], st["m"], rtol=1e-5, atol=1e-4)
        assert np.allclose(rest[rows], st["rest"], rtol=1e-3)
        scale = np.abs(st["a"]).max()
        assert np.allclose(a[rows], st["a"], rtol=2e-2, atol=2e-3 * scale)


def _dominant_case(gaps, n=700, w=4, G=2, seed=0):
    """One KV head; row t*w+i gets a planted key whose logit exceeds the rest by gaps[row]."""
    d = 128
    rng = np.random.default_rng(seed)
    rows = G * w
    assert len(gaps) == rows
    q = np.zeros((G, w, d), np.float32)
    k = (rng.standard_normal((1, n, d)) * 0.05).astype(np.float32)
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    # row r uses its own coordinate axis r; its planted key sits at position 10 + 7r
    for r in range(rows):
        t, i = divmod(r, w)
        q[t, i, r] = 1.0
        k[0, 10 + 7 * r, r] = gaps[r] * math.sqrt(d)
    to_bf = synth.bf16_round_bits
    return synth.Case(q=to_bf(q), k=to_bf(k), v=to_bf(v), n=n, window=w, Hq=G, Hkv=1, d=d, dtype="bf16")


def test_mfma_flagged_rows_match_oracle():
    """Rows with p_max between 1/2 and 1 - 1e-6 take the exact argmax fix-up."""
    gaps = [0.0, 2.0, 7.0, 8.0, 10.0, 13.0, 16.0, 20.0]
    case = _dominant_case(gaps)
    ref = run_oracle(case, 3, 100)
    rests = np.concatenate([st["rest"] for st in ref["stats"]])
    assert rests.min() < 1e-5 and rests.max() > 1.0  # both kinds of rows present
    _compare(case, 3, 100, "flagged")
    q, k, v = to_torch(case)
    m, rest, arg, a = (t.cpu().numpy() for t in K.row_stats(q, k, v))
    jst = np.concatenate([st["jstar"] for st in ref["stats"]])
    fl = rests < 1.0
    assert np.array_equal(arg[fl], jst[fl])
    assert np.allclose(rest[fl], rests[fl], rtol=2e-2)


@pytest.mark.parametrize("pool", [1, 1031])
def test_mfma_flagged_rows_pool_widths(pool):
    """The argmax terms reach the pooled scores both when the pool stage folds
    them into its LDS tile and when a pool wider than that tile folds them first."""
    gaps = [0.0, 2.0, 7.0, 8.0, 10.0, 13.0, 16.0, 20.0]
    case = _dominant_case(gaps, n=3000, seed=3)
    _compare(case, pool, 1500, f"flagged pool={pool}")


@pytest.mark.parametrize("n", [300, 3000])
def test_mfma_flagged_rows_wide_group(n):
    """40 window rows per KV head (two row blocks): the argmax fix-up of the
    flagged rows runs inside pass 2's workgroups, also when the head has fewer
    tiles than fix-up chunks (n = 300: five workgroups cover eight chunks)."""
    gaps = [0.0, 2.0, 7.0, 8.0, 10.0, 13.0, 16.0, 20.0] * 5
    case = _dominant_case(gaps, n=n, w=20, G=2, seed=5)
    ref = run_oracle(case, 3, 100)
    rests = np.concatenate([st["rest"] for st in ref["stats"]])
    assert rests.min() < 1e-5 and rests.max() > 1.0  # both kinds of rows present
    _compare(case, 3, (n - 20) // 2, f"flagged wide n={n}")


def test_mfma_singular_row_rejected():
    gaps = [0.0, 2.0, 30.0, 1.0, 0.5, 0.0, 3.0, 1.0]  # gap 30 -> R ~ 700 e^-30 < 2^-24
    case = _dominant_case(gaps)
    with pytest.raises(oracle.SingularRow):
        run_oracle(case, 3, 10)
    q, k, v = to_torch(case)
    with pytest.raises(K.DropKVSingularError):
        K.score(q, k, v, pool_kernel=3, n_evict=10)


def test_mfma_matches_generic_path():
    case = synth.make_gaussian_case(16, 4, 128, 2500, 32, dtype="bf16", seeds=(9, 9, 9), sink=True, needles=8)
    q, k, v = to_torch(case)
    S_mfma = K.raw_scores(q, k, v).cpu().numpy()
    S_gen = K.raw_scores(q, k, v, flags=K.FLAG_GENERIC).cpu().numpy()
    assert max_rel_err(S_mfma, S_gen) <= RTOL["bf16"]


def test_mfma_nan_in_values_reported():
    case = synth.make_gaussian_case(8, 2, 128, 500, 8, dtype="bf16", seeds=(1, 2, 3))
    case.v[1, 77, 5] = 0x7FC0  # bf16 quiet NaN
    q, k, v = to_torch(case)
    with pytest.raises(K.DropKVNonFiniteError):
        K.score(q, k, v, pool_kernel=3, n_evict=100)


def test_stage_log_over_async_calls():
    """Logged dropkv_score_ex calls report every kernel's mean time, in order, and match unlogged outputs."""
    case = synth.make_gaussian_case(8, 2, 128, 3000, 32, dtype="bf16", seeds=(5, 6, 7), sink=True, needles=4)
    print(f"[mfma] stage log Hq={case.Hq} Hkv={case.Hkv} n={case.n}", flush=True)
    q, k, v = to_torch(case)
    ne = 2000
    ws = torch.empty(K.workspace_bytes(K.BF16, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device=q.device)
    st = torch.zeros(1, dtype=torch.int32, device=q.device)
    K.stage_log()
    ref_scores, ref_idx = K.score(q, k, v, pool_kernel=7, n_evict=ne)
    outs = []
    for _ in range(3):
        outs.append(K.score_ex(q, k, v, pool_kernel=7, n_evict=ne, workspace=ws, status=st,
                               flags=K.FLAG_STAGE_LOG))
    calls, stages = K.stage_log()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert calls == 3
    names = [s for s, _ in stages]
    assert names[0] == "pass1" and names[-1] == "select" and "pass2" in names
    assert all(ms > 0 for _, ms in stages)
    for sc, ix in outs:
        assert torch.equal(sc, ref_scores) and torch.equal(ix, ref_idx)
    assert K.stage_log() == (0, [])
