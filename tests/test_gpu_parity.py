"""HIP library vs the fp64 oracle, element by element, through the C ABI.

Every test here needs an MI355X and the built libdropkv.so; the library must
be the code that runs (no fallback exists).
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


def _gpu_run(case, pool_kernel, n_evict, flags=0):
    q, k, v = to_torch(case)
    if flags:
        ws = torch.empty(K.workspace_bytes(0 if case.dtype == "bf16" else 1, case.n, case.window,
                                           case.Hq, case.Hkv, case.d), dtype=torch.uint8, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        scores, idx = K.score_ex(q, k, v, pool_kernel=pool_kernel, n_evict=n_evict, workspace=ws,
                                 status=st, flags=flags)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
    else:
        scores, idx = K.score(q, k, v, pool_kernel=pool_kernel, n_evict=n_evict)
    S = K.raw_scores(q, k, v, flags=flags)
    return scores.cpu().numpy(), idx.cpu().numpy(), S.cpu().numpy()


def _check_case(case, pool_kernel, n_evict, flags=0, min_exact=0):
    rtol = RTOL[case.dtype]
    print(f"case Hq={case.Hq} Hkv={case.Hkv} d={case.d} n={case.n} w={case.window} "
          f"dtype={case.dtype} k={pool_kernel} evict={n_evict} flags={flags}", flush=True)
    scores, idx, S = _gpu_run(case, pool_kernel, n_evict, flags)
    ref = run_oracle(case, pool_kernel, n_evict)
    e_S = max_rel_err(S, ref["S"])
    e_P = max_rel_err(scores, ref["P"])
    assert e_S <= rtol, f"raw scores rel err {e_S:.3e} > {rtol}"
    assert e_P <= rtol, f"pooled scores rel err {e_P:.3e} > {rtol}"
    exact, jac = check_evictions(scores, idx, ref["P"], ref["S"], ref["evict"], n_evict, rtol)
    assert exact >= min_exact
    return e_S, exact, jac


# ------------------------------------------------------------------ tiny case ---

def _tiny_cases(dtype):
    cfg = synth.CONFIGS["tiny"]
    out = [synth.make_case(cfg, one_stream_seed=s, dtype=dtype) for s in cfg.seeds]
    out.append(synth.make_case(cfg, dtype=dtype))
    return out


@pytest.mark.parametrize("ci", range(4))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_protocol(ci, dtype):
    case = _tiny_cases(dtype)[ci]
    _check_case(case, pool_kernel=3, n_evict=7)


# ---------------------------------------------------------- ragged / odd shapes ---

RAGGED = [
    # Hq, Hkv, d, n, w, dtype, pool, n_evict
    (1, 1, 4, 2, 1, "f32", 1, 1),        # n = w + 1
    (2, 1, 8, 3, 2, "f32", 3, 1),
    (8, 8, 16, 255, 3, "f32", 5, 100),    # G = 1
    (7, 1, 32, 257, 32, "bf16", 7, 200),  # G = 7
    (8, 2, 64, 300, 64, "bf16", 3, 236),  # evict everything unprotected
    (4, 2, 128, 1000, 1, "bf16", 7, 0),   # w = 1, nothing evicted
    (16, 2, 128, 4097, 32, "bf16", 7, 3000),  # G = 8, ragged tail
    (4, 1, 256, 513, 5, "f32", 9, 50),    # d = 256
    (4, 2, 100, 700, 9, "f32", 3, 333),   # d not a power of two
]


@pytest.mark.parametrize("spec", RAGGED, ids=[str(r[:5]) for r in RAGGED])
def test_ragged_shapes(spec):
    Hq, Hkv, d, n, w, dtype, pool, ne = spec
    case = synth.make_gaussian_case(Hq, Hkv, d, n, w, dtype=dtype, seeds=(7, 8, 9),
                                    sink=n > w + 2, needles=min(4, max(0, n - w - 2)))
    _check_case(case, pool, ne)


# ------------------------------------------------------- Llama 4K layer, full ---

def test_llama_4k_full():
    cfg = synth.CONFIGS["llama_4k"]
    case = synth.make_case(cfg)
    e_S, exact, jac = _check_case(case, cfg.pool_kernel, cfg.n_evicts()[0])
    print(f"llama_4k: rel err {e_S:.2e}, exact heads {exact}/8, jaccard min {min(jac):.4f}")


def test_generic_flag_matches_default_path():
    case = synth.make_gaussian_case(8, 2, 128, 1500, 32, dtype="bf16", seeds=(3, 4, 5),
                                    sink=True, needles=8)
    _check_case(case, 7, 1000, flags=K.FLAG_GENERIC)
    _check_case(case, 7, 1000, flags=0)


# ----------------------------------------------------------------- row stats ---

def test_row_stats_match_oracle():
    case = synth.make_gaussian_case(4, 2, 16, 200, 6, dtype="f32", seeds=(1, 2, 3), sink=True, needles=3)
    q, k, v = to_torch(case)
    m, rest, arg, a = (t.cpu().numpy() for t in K.row_stats(q, k, v, flags=K.FLAG_GENERIC))
    qf, kf, vf = (oracle.as_f64(t, "f32") for t in (case.q, case.k, case.v))
    G = case.group
    for g in range(case.Hkv):
        st = oracle.head_row_stats(qf, kf, vf, g, G, case.n, case.window)
        rows = slice(g * G * case.window, (g + 1) * G * case.window)
        assert np.allclose(m[rows], st["m"], rtol=1e-5, atol=1e-6)
        assert np.allclose(rest[rows], st["rest"], rtol=1e-5)
        assert np.array_equal(arg[rows], st["jstar"])
        assert np.allclose(a[rows], st["a"], rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------ determinism ---

def test_bitwise_repeatable():
    case = synth.make_gaussian_case(8, 2, 128, 3000, 32, dtype="bf16", seeds=(5, 6, 7), sink=True, needles=8)
    a = _gpu_run(case, 7, 2000)
    b = _gpu_run(case, 7, 2000)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


# ------------------------------------------------------------ select stage ---

@pytest.mark.parametrize("n,w,k,ne", [(50, 6, 3, 20), (4097, 64, 7, 3000), (1000, 10, 1, 990),
                                      (300, 5, 5, 0), (64, 1, 3, 63),
                                      # thousands of keys tied with tau: candidates beyond the
                                      # on-chip buffer, ties beyond the tie list
                                      (40000, 64, 7, 30000),
                                      # segments of 24 keys: several load groups per segment and
                                      # workgroups with more evictions than their staging area
                                      (300000, 64, 9, 250000),
                                      # either side of the largest head selected inside one
                                      # workgroup (32768 keys), and every evictable token evicted
                                      (32768, 64, 7, 31130), (32769, 64, 7, 31131), (20000, 16, 3, 19984),
                                      # either side of the heads selected by one workgroup in LDS
                                      # (<= 4096 keys, pooling half-width <= 32)
                                      (4096, 64, 7, 3000), (4096, 16, 65, 4000), (4096, 16, 67, 100),
                                      (4095, 32, 1, 4063), (22, 3, 3, 7)])
def test_select_matches_stable_argsort(n, w, k, ne):
    rng = np.random.default_rng(n + ne)
    S = rng.integers(0, 7, size=(3, n)).astype(np.float32) * np.float32(0.25)  # many exact ties
    S[1] = rng.random(n).astype(np.float32)
    S[2, : n // 2] = 0.0
    P_ref = oracle.protect_window(oracle.maxpool1d_same(S.astype(np.float64), k), w)
    ev_ref = oracle.evict_smallest(P_ref, ne)
    scores, idx = K.select(torch.from_numpy(S).cuda(), window=w, pool_kernel=k, n_evict=ne)
    scores, idx = scores.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(scores.astype(np.float64), P_ref)
    assert np.array_equal(idx, ev_ref)


@pytest.mark.parametrize("n", [4096, 32768, 32769])
def test_select_all_keys_tied(n):
    """Every pooled score equal: tau is that value and the lowest indices are evicted."""
    S = np.full((2, n), 0.5, np.float32)
    ne = n // 2 + 3
    scores, idx = K.select(torch.from_numpy(S).cuda(), window=8, pool_kernel=5, n_evict=ne)
    P_ref = oracle.protect_window(oracle.maxpool1d_same(S.astype(np.float64), 5), 8)
    assert np.array_equal(scores.cpu().numpy().astype(np.float64), P_ref)
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(ne, dtype=np.int64), (2, 1)))


@pytest.mark.parametrize("n,where", [(9001, 0), (9001, 4095), (9001, 9000), (4000, 0), (4000, 3999)])
def test_select_rejects_negative_scores(n, where):
    """Given raw scores must be >= 0 (sums of squared norms): a negative entry
    anywhere is reported; -0.0 is accepted and orders as +0 (on the
    three-kernel stage and on the one-workgroup stage of short heads)."""
    w, k, ne = 16, 7, 500
    rng = np.random.default_rng(where)
    S = rng.random((2, n)).astype(np.float32)
    S[1, where] = -1e-30
    with pytest.raises(K.DropKVNegativeScoreError):
        K.select(torch.from_numpy(S).cuda(), window=w, pool_kernel=k, n_evict=ne)
    S[1, where] = -0.0
    P_ref = oracle.protect_window(oracle.maxpool1d_same(np.abs(S.astype(np.float64)), k), w)
    scores, idx = K.select(torch.from_numpy(S).cuda(), window=w, pool_kernel=k, n_evict=ne)
    assert np.array_equal(idx.cpu().numpy(), oracle.evict_smallest(P_ref, ne))


@pytest.mark.parametrize("n", [4000, 9000])
def test_select_reports_nan_scores(n):
    """A NaN among given raw scores is reported (pooling would otherwise hide
    it), on both select stages."""
    S = np.random.default_rng(n).random((2, n)).astype(np.float32)
    S[1, n // 2] = np.nan
    with pytest.raises(K.DropKVNonFiniteError):
        K.select(torch.from_numpy(S).cuda(), window=16, pool_kernel=7, n_evict=100)


def test_pass1_stats_name_matches_row_stats():
    case = synth.make_case(synth.CONFIGS["llama_4k"])
    q, k, v = to_torch(case)
    a = K.row_stats(q, k, v)
    b = K.pass1_stats(q, k, v)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------------------ failure paths ---

def test_singular_row_rejected():
    rng = np.random.default_rng(31)
    Hq, Hkv, d, n, w = 2, 1, 8, 16, 2
    q = rng.standard_normal((Hq, w, d)).astype(np.float32)
    k = (rng.standard_normal((Hkv, n, d)) * 0.1).astype(np.float32)
    v = rng.standard_normal((Hkv, n, d)).astype(np.float32)
    u = q[1, 0] / np.linalg.norm(q[1, 0])
    k[0, 5] = (80.0 * math.sqrt(d) / np.linalg.norm(q[1, 0]) * u).astype(np.float32)
    case = synth.Case(q=q, k=k, v=v, n=n, window=w, Hq=Hq, Hkv=Hkv, d=d, dtype="f32")
    with pytest.raises(oracle.SingularRow):
        run_oracle(case, 1, 0)
    qt, kt, vt = to_torch(case)
    with pytest.raises(K.DropKVSingularError):
        K.score(qt, kt, vt, pool_kernel=1, n_evict=0)


def test_nan_input_reported():
    case = synth.make_gaussian_case(4, 2, 16, 64, 4, dtype="f32", seeds=(1, 2, 3))
    case.k[1, 10, 3] = np.nan
    q, k, v = to_torch(case)
    with pytest.raises(K.DropKVNonFiniteError):
        K.score(q, k, v, pool_kernel=3, n_evict=10)


def test_invalid_call_leaves_outputs_untouched():
    case = synth.make_gaussian_case(4, 2, 16, 64, 4, dtype="f32", seeds=(1, 2, 3))
    q, k, v = to_torch(case)
    lib = K.load_library()
    out = torch.full((2, 64), 7.0, device="cuda")
    idx = torch.full((2, 70), -5, dtype=torch.int64, device="cuda")
    rc = lib.dropkv_score_f32(q.data_ptr(), k.data_ptr(), v.data_ptr(), 64, 4, 4, 2, 16, 3, 70,
                              out.data_ptr(), idx.data_ptr(), None)
    assert rc == -1
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(idx == -5)
    # host memory for an input is rejected, not dereferenced
    host = np.zeros(4 * 4 * 16, np.float32)
    rc = lib.dropkv_score_f32(host.ctypes.data, k.data_ptr(), v.data_ptr(), 64, 4, 4, 2, 16, 3, 10,
                              out.data_ptr(), idx.data_ptr(), None)
    assert rc == -1


def test_score_ex_async_matches_sync():
    case = synth.make_gaussian_case(8, 4, 128, 2000, 16, dtype="bf16", seeds=(11, 12, 13), sink=True, needles=4)
    q, k, v = to_torch(case)
    s1, i1 = K.score(q, k, v, pool_kernel=5, n_evict=1500)
    ws = torch.empty(K.workspace_bytes(0, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device="cuda")
    st = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    s2, i2 = K.score_ex(q, k, v, pool_kernel=5, n_evict=1500, workspace=ws, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(s1, s2) and torch.equal(i1, i2)
