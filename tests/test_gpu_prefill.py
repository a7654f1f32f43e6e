"""Prefill attention with handed-over scoring statistics (dropkv_prefill_attention).

The output o of every position is compared with the fp64 oracle's attention
output at that position (all rows on small layers, sampled rows on larger
ones); the window rows' statistics with the scoring oracle's row statistics;
and the whole producer -> consumer path (prefill statistics into
dropkv_score_from_stats) with the oracle's DropKV scores and evicted sets,
and with dropkv_score's own outputs.
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

# o is stored in bf16 (relative rounding 2^-9) after a product with bf16
# probabilities (2^-9 per weight): compared per row against 1e-2 of the row's
# largest |o|, well above both and far below any real mistake.
O_TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    yield


def _bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run(case, qa):
    q_all = torch.from_numpy(qa.view(np.int16).copy()).view(torch.bfloat16).cuda().contiguous()
    _, k, v = to_torch(case)
    st = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    o, m, rest, arg, a = K.prefill_attention(q_all, k, v, window=case.window, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, f"device status {int(st.item())}"
    return q_all, k, v, o, m, rest, arg, a


def _check_o(case, qa, o, rows):
    ref = oracle.prefill_outputs(qa, case.k, case.v, rows, Hq=case.Hq, Hkv=case.Hkv, dtype=case.dtype)
    got = _bf16_to_f64(o)
    worst = 0.0
    for r, (h, pos) in enumerate(rows):
        scale = max(np.max(np.abs(ref[r])), 1e-6)
        err = np.max(np.abs(got[h, pos] - ref[r])) / scale
        worst = max(worst, err)
        assert err <= O_TOL, f"o(head {h}, position {pos}): error {err:.3e} of the row's largest |o|"
    return worst


def _check_stats(case, m, rest, arg, a):
    qf, kf, vf = (oracle.as_f64(t, case.dtype) for t in (case.q, case.k, case.v))
    G = case.group
    m, rest, arg, a = (t.cpu().numpy() for t in (m, rest, arg, a))
    for g in range(case.Hkv):
        st = oracle.head_row_stats(qf, kf, vf, g, G, case.n, case.window)
        sl = slice(g * G * case.window, (g + 1) * G * case.window)
        assert np.max(np.abs(m[sl] - st["m"]) / np.maximum(np.abs(st["m"]), 1.0)) <= 1e-3
        # R: relative for R >= 1; absolute 1e-3 below (R is formed as L - 1 there)
        assert np.max(np.abs(rest[sl] - st["rest"]) / np.maximum(st["rest"], 1.0)) <= 2e-3
        small = st["rest"] < 1.0
        assert np.array_equal(arg[sl][small], st["jstar"][small]), "argmax of rows with p_max > 1/2"
        scale = np.maximum(np.max(np.abs(st["a"]), axis=1, keepdims=True), 1e-6)
        assert np.max(np.abs(a[sl] - st["a"]) / scale) <= 5e-3


def _end_to_end(case, q, k, v, m, rest, arg, a, pool, ne, oracle_ref=True):
    sc, idx = K.score_from_stats(q, k, v, m, rest, arg, a, pool_kernel=pool, n_evict=ne)
    base_sc, base_idx = K.score(q, k, v, pool_kernel=pool, n_evict=ne)
    sc, idx, base_sc = sc.cpu().numpy(), idx.cpu().numpy(), base_sc.cpu().numpy()
    assert max_rel_err(sc, base_sc) <= 5e-3
    if oracle_ref:
        ref = run_oracle(case, pool, ne)
        assert max_rel_err(sc, ref["P"]) <= RTOL["bf16"]
        check_evictions(sc, idx, ref["P"], ref["S"], ref["evict"], ne, RTOL["bf16"])


@pytest.mark.parametrize("n,w,Hq,Hkv", [(257, 5, 4, 1), (1000, 32, 8, 2), (700, 64, 28, 4), (520, 3, 16, 1),
                                        (300, 17, 6, 6)])
def test_prefill_small_layers_all_rows(n, w, Hq, Hkv):
    case = synth.make_gaussian_case(Hq, Hkv, 128, n, w, dtype="bf16", seeds=(n, w, 5), sink=True, needles=4)
    qa = synth.prefill_queries(case, seed=n + 1)
    print(f"[prefill] Hq={Hq} Hkv={Hkv} n={n} w={w}", flush=True)
    q_all, k, v, o, m, rest, arg, a = _run(case, qa)
    rows = [(h, p) for h in range(Hq) for p in range(n)]
    worst = _check_o(case, qa, o, rows)
    print(f"[prefill] worst o error {worst:.2e}", flush=True)
    _check_stats(case, m, rest, arg, a)
    q, _, _ = to_torch(case)
    _end_to_end(case, q, k, v, m, rest, arg, a, 7, (n - w) // 2)


def test_prefill_flagged_rows_end_to_end():
    """Window rows with p_max > 1/2 (planted dominant keys): exact argmax handed over,
    and the consumer's fix-up gives the oracle's scores."""
    d, n, w, G = 128, 1500, 4, 2
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
    qa = synth.prefill_queries(case, seed=3)
    q_all, kk, vv, o, m, rest, arg, a = _run(case, qa)
    _check_stats(case, m, rest, arg, a)
    qt, _, _ = to_torch(case)
    _end_to_end(case, qt, kk, vv, m, rest, arg, a, 3, 700)


def test_prefill_llama_4k_layer():
    cfg = synth.CONFIGS["llama_4k"]
    case = synth.make_case(cfg)
    qa = synth.prefill_queries(case, seed=4242)
    print(f"[prefill] llama_4k n={case.n}", flush=True)
    q_all, k, v, o, m, rest, arg, a = _run(case, qa)
    rng = np.random.default_rng(9)
    rows = [(int(h), int(p)) for h, p in zip(rng.integers(0, case.Hq, 300), rng.integers(0, case.n, 300))]
    rows += [(h, p) for h in (0, 31) for p in (0, 1, 63, 64, case.n - case.window - 1, case.n - 1)]
    _check_o(case, qa, o, rows)
    _check_stats(case, m, rest, arg, a)
    q, _, _ = to_torch(case)
    _end_to_end(case, q, k, v, m, rest, arg, a, cfg.pool_kernel, cfg.n_evicts()[0])


def test_prefill_llama_32k_layer_sampled():
    cfg = synth.CONFIGS["llama_32k"]
    case = synth.make_case(cfg)
    qa = synth.prefill_queries(case, seed=4343)
    print(f"[prefill] llama_32k n={case.n}", flush=True)
    q_all, k, v, o, m, rest, arg, a = _run(case, qa)
    rng = np.random.default_rng(10)
    rows = [(int(h), int(p)) for h, p in zip(rng.integers(0, case.Hq, 64), rng.integers(0, case.n, 64))]
    rows += [(h, case.n - 1 - i) for h in (3, 30) for i in (0, 1, 63)]
    _check_o(case, qa, o, rows)
    q, _, _ = to_torch(case)
    _end_to_end(case, q, k, v, m, rest, arg, a, cfg.pool_kernel, cfg.n_evicts()[0], oracle_ref=False)


def test_prefill_rejects_bad_arguments():
    case = synth.make_gaussian_case(8, 2, 128, 300, 8, dtype="bf16", seeds=(1, 2, 3))
    qa = synth.prefill_queries(case, seed=1)
    q_all = torch.from_numpy(qa.view(np.int16).copy()).view(torch.bfloat16).cuda()
    _, k, v = to_torch(case)
    with pytest.raises(K.DropKVInvalidError):
        K.prefill_attention(q_all, k, v, window=300)  # window must be below n
    with pytest.raises(K.DropKVInvalidError):
        K.prefill_attention(q_all[:, :200].contiguous(), k, v, window=8)  # n disagrees


def test_prefill_llama_128k_layer_sampled():
    """The headline layer: o on sampled rows (the sink's neighbourhood, the window, random
    positions), the window statistics of every head, and scoring from them against the
    two-pass scoring step."""
    cfg = synth.CONFIGS["llama_128k"]
    case = synth.make_case(cfg)
    qa = synth.prefill_queries(case, seed=cfg.seeds[0] + 7)
    print(f"[prefill] llama_128k n={case.n}", flush=True)
    q_all, k, v, o, m, rest, arg, a = _run(case, qa)
    rng = np.random.default_rng(12)
    rows = [(int(h), int(p)) for h, p in zip(rng.integers(0, case.Hq, 24), rng.integers(0, case.n, 24))]
    rows += [(h, p) for h in (0, 17) for p in (0, 1, 4095, 4096, case.n - case.window, case.n - 1)]
    _check_o(case, qa, o, rows)
    del q_all, o
    _check_stats(case, m, rest, arg, a)
    q, _, _ = to_torch(case)
    _end_to_end(case, q, k, v, m, rest, arg, a, cfg.pool_kernel, cfg.n_evicts()[0], oracle_ref=False)
