"""The full-size workloads against the fp64 oracle, in the benchmark's launch configuration.

Every call goes through dropkv_score_ex with a caller-owned workspace, as the
benchmark times it. Every KV head of every workload is compared with the
oracle in full: raw scores S, pooled scores P and the evicted set, the last
under all of check_evictions' rules (own bottom-k, the k-th / (k+1)-th gap
rule, the plateau rule, and the error band that every differing index must
fall in). The GPU runs once per workload (module fixtures); the oracle runs
one KV head per test, so each test stays short.
"""

import numpy as np
import pytest

import oracle
import kv_cache_eviction_pass1_amd as K
from kv_cache_eviction_pass1_amd import synth
from parity import RTOL, check_evictions, max_rel_err, own_bottom_k, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

QWEN_LAYERS = [(0, 0), (1, 27)]  # (sequence b, layer l) of the 28-layer, 2-sequence sweep


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    yield


def _run_ex(case, pool, n_evict):
    q, k, v = to_torch(case)
    dcode = K.BF16 if case.dtype == "bf16" else K.F32
    ws = torch.empty(K.workspace_bytes(dcode, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    scores, idx = K.score_ex(q, k, v, pool_kernel=pool, n_evict=n_evict, workspace=ws, status=st)
    S = K.raw_scores(q, k, v)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, f"device status {int(st.item())}"
    out = scores.cpu().numpy(), idx.cpu().numpy(), S.cpu().numpy()
    del q, k, v, ws, st, scores, idx, S
    torch.cuda.empty_cache()
    return out


def _check_protection_and_own_bottom_k(case, P, idx, n_evict):
    n, w = case.n, case.window
    assert np.all(np.isinf(P[:, n - w:])) and np.all(np.isfinite(P[:, : n - w]))
    for g in range(case.Hkv):
        assert np.array_equal(idx[g], own_bottom_k(P[g], n_evict)), f"head {g}: not its own bottom-k"
        assert idx[g].max() < n - w


def _check_head(tag, case, pool, ne, P, idx, S, g):
    """One KV head in full against the oracle: S, P and the evicted set."""
    ref = oracle.dropkv_oracle(case.q, case.k, case.v, n=case.n, window=case.window, Hq=case.Hq,
                               Hkv=case.Hkv, d=case.d, pool_kernel=pool, n_evict=ne,
                               dtype=case.dtype, heads=[g])
    e_S = max_rel_err(S[g:g + 1], ref["S"])
    e_P = max_rel_err(P[g:g + 1], ref["P"])
    assert e_S <= RTOL["bf16"], f"{tag} head {g}: raw scores rel err {e_S:.3e}"
    assert e_P <= RTOL["bf16"], f"{tag} head {g}: pooled scores rel err {e_P:.3e}"
    rep = {}
    exact, jac = check_evictions(P[g:g + 1], idx[g:g + 1], ref["P"], ref["S"], ref["evict"], ne,
                                 RTOL["bf16"], report=rep)
    print(f"[full] {tag} head {g}: S err {e_S:.2e} P err {e_P:.2e} exact {exact} "
          f"(gap {rep['gap_exact']}, plateau {rep['plateau_exact']}, band {rep['band_checked']}) "
          f"symdiff {rep['symdiff_max']} band used {rep['band_used_max']:.2e} jaccard {jac[0]:.6f}",
          flush=True)
    return rep


@pytest.fixture(scope="module")
def llama_128k():
    cfg = synth.CONFIGS["llama_128k"]
    case = synth.make_case(cfg)
    ne = cfg.n_evicts()[0]
    print(f"[full] llama_128k n={case.n} evict={ne}", flush=True)
    P, idx, S = _run_ex(case, cfg.pool_kernel, ne)
    _check_protection_and_own_bottom_k(case, P, idx, ne)
    return cfg, case, ne, P, idx, S


@pytest.fixture(scope="module")
def qwen_layers():
    cfg = synth.CONFIGS["qwen_128k_sweep"]
    ne = cfg.n_evicts()[0]
    out = {}
    for b, layer in QWEN_LAYERS:
        case = synth.make_case(cfg, layer=layer, b=b)
        print(f"[full] qwen_128k b={b} layer={layer}: Hq={case.Hq} Hkv={case.Hkv} n={case.n} evict={ne}",
              flush=True)
        P, idx, S = _run_ex(case, cfg.pool_kernel, ne)
        _check_protection_and_own_bottom_k(case, P, idx, ne)
        out[(b, layer)] = (case, P, idx, S)
    return cfg, ne, out


def test_llama_32k_full_both_budgets():
    cfg = synth.CONFIGS["llama_32k"]
    case = synth.make_case(cfg)
    ref = None
    for ne in cfg.n_evicts():
        print(f"[full] llama_32k n={case.n} evict={ne}", flush=True)
        P, idx, S = _run_ex(case, cfg.pool_kernel, ne)
        if ref is None:
            ref = oracle.dropkv_oracle(case.q, case.k, case.v, n=case.n, window=case.window,
                                       Hq=case.Hq, Hkv=case.Hkv, d=case.d,
                                       pool_kernel=cfg.pool_kernel, n_evict=ne, dtype=case.dtype)
            assert max_rel_err(S, ref["S"]) <= RTOL["bf16"]
            assert max_rel_err(P, ref["P"]) <= RTOL["bf16"]
        ref_idx = oracle.evict_smallest(ref["P"], ne)
        _check_protection_and_own_bottom_k(case, P, idx, ne)
        rep = {}
        exact, jac = check_evictions(P, idx, ref["P"], ref["S"], ref_idx, ne, RTOL["bf16"], report=rep)
        print(f"[full] llama_32k evict={ne}: exact heads {exact}/8 (gap {rep['gap_exact']}, "
              f"plateau {rep['plateau_exact']}), band-checked {rep['band_checked']}, "
              f"largest symdiff {rep['symdiff_max']}, jaccard min {min(jac):.5f}", flush=True)
        assert rep["heads"] == 8 and rep["gap_exact"] + rep["plateau_exact"] + rep["band_checked"] == 8


@pytest.mark.parametrize("g", range(8))
def test_llama_128k_head(llama_128k, g):
    cfg, case, ne, P, idx, S = llama_128k
    rep = _check_head("llama_128k", case, cfg.pool_kernel, ne, P, idx, S, g)
    assert rep["gap_exact"] + rep["plateau_exact"] + rep["band_checked"] == 1


@pytest.mark.parametrize("bl", QWEN_LAYERS, ids=[f"b{b}_l{l}" for b, l in QWEN_LAYERS])
@pytest.mark.parametrize("g", range(4))
def test_qwen_128k_head(qwen_layers, bl, g):
    cfg, ne, out = qwen_layers
    case, P, idx, S = out[bl]
    rep = _check_head(f"qwen_128k b={bl[0]} l={bl[1]}", case, cfg.pool_kernel, ne, P, idx, S, g)
    assert rep["gap_exact"] + rep["plateau_exact"] + rep["band_checked"] == 1
