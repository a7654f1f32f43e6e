"""The full-size workloads against the fp64 oracle, in the benchmark's launch configuration.

Every call goes through dropkv_score_ex with a caller-owned workspace, as the
benchmark times it. At 32K the oracle runs in full; at 128K it runs in full
for one KV head (exact eviction set) and on sampled tokens elsewhere (the
sink, the needles, pass-1 chunk edges, the window edge, the ragged end and
random tokens, each with its pooling neighbours). On every head the evicted
set must be the bottom-n_evict of the GPU's own pooled scores.
"""

import numpy as np
import pytest

import oracle
import kv_cache_eviction_pass1_amd as K
from kv_cache_eviction_pass1_amd import synth
from parity import RTOL, check_evictions, check_sampled, max_rel_err, own_bottom_k, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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
    return scores.cpu().numpy(), idx.cpu().numpy(), S.cpu().numpy()


def _check_protection_and_own_bottom_k(case, P, idx, n_evict):
    n, w = case.n, case.window
    assert np.all(np.isinf(P[:, n - w:])) and np.all(np.isfinite(P[:, : n - w]))
    for g in range(case.Hkv):
        assert np.array_equal(idx[g], own_bottom_k(P[g], n_evict)), f"head {g}: not its own bottom-k"
        assert idx[g].max() < n - w


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
        exact, jac = check_evictions(P, idx, ref["P"], ref["S"], ref_idx, ne, RTOL["bf16"])
        print(f"[full] llama_32k evict={ne}: exact heads {exact}/8, jaccard min {min(jac):.5f}")
        assert min(jac) > 0.99


def test_llama_128k_headline_layer():
    cfg = synth.CONFIGS["llama_128k"]
    case = synth.make_case(cfg)
    ne = cfg.n_evicts()[0]
    print(f"[full] llama_128k n={case.n} evict={ne}", flush=True)
    P, idx, S = _run_ex(case, cfg.pool_kernel, ne)
    _check_protection_and_own_bottom_k(case, P, idx, ne)
    rng = np.random.default_rng(2024)
    for g in (3, 7):
        check_sampled(case, g, cfg.pool_kernel, S, P, rng)
    # head 0 in full: scores and the exact evicted set
    ref = oracle.dropkv_oracle(case.q, case.k, case.v, n=case.n, window=case.window, Hq=case.Hq,
                               Hkv=case.Hkv, d=case.d, pool_kernel=cfg.pool_kernel, n_evict=ne,
                               dtype=case.dtype, heads=[0])
    assert max_rel_err(S[:1], ref["S"]) <= RTOL["bf16"]
    assert max_rel_err(P[:1], ref["P"]) <= RTOL["bf16"]
    exact, jac = check_evictions(P[:1], idx[:1], ref["P"], ref["S"], ref["evict"], ne, RTOL["bf16"])
    print(f"[full] llama_128k head 0: exact {exact}, jaccard {jac[0]:.6f}")
    assert jac[0] > 0.999


def test_qwen_128k_layer_sampled():
    cfg = synth.CONFIGS["qwen_128k_sweep"]
    case = synth.make_case(cfg, layer=27, b=1)
    ne = cfg.n_evicts()[0]
    print(f"[full] qwen_128k layer 27 b 1: Hq={case.Hq} Hkv={case.Hkv} n={case.n} evict={ne}", flush=True)
    P, idx, S = _run_ex(case, cfg.pool_kernel, ne)
    _check_protection_and_own_bottom_k(case, P, idx, ne)
    rng = np.random.default_rng(2025)
    for g in (0, 3):
        check_sampled(case, g, cfg.pool_kernel, S, P, rng)
