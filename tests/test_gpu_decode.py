"""Decode-time rescoring on the GPU (dropkv_decode_*) against the oracle.

The cache grows token by token from a scored prefix; after the first scoring
and after every checked step, the kept raw score must match the oracle's
score of the grown cache computed from scratch (relative 2e-2, bf16 inputs),
including after more steps than the window holds (every prefix row has left),
and at the full 128K layer in the benchmark's launch configuration.
The fp64 score kept incrementally must equal a rebuild from the stored window
rows to fp64 rounding (the subtracted terms are bit for bit the added ones),
re-eviction must equal the select stage on the same raw score and the oracle's
eviction where the gap rule allows, and invalid calls / singular rows are
reported. The single-pass (deferred) step must give the two-pass step's score
once its pending terms are flushed, in any mix with two-pass steps, flushes
and rebuilds.
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


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


def _setup(Hq, Hkv, n0, w, steps, n_max, needles=4, seeds=(42, 43, 44)):
    d = 128
    q_all, k, v = synth.make_decode_case(Hq, Hkv, d, n0 + steps, seeds=seeds, needles=needles)
    kc = torch.zeros((Hkv, n_max, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, : n0 + steps] = _dev(k)
    vc[:, : n0 + steps] = _dev(v)
    sc = K.DecodeScorer(n_max=n_max, window=w, Hq=Hq, Hkv=Hkv, d=d)
    sc.init(_dev(q_all[:, n0 - w:n0]).contiguous(), kc, vc, n0)
    return sc, q_all, k, v, kc, vc


def _ref(q_all, k, v, n, w, Hq, Hkv):
    return oracle.decode_scratch(q_all[:, n - w:n], k, v, n=n, window=w, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16")


@pytest.mark.parametrize("Hq,Hkv,n0,w,steps,n_max,check_every", [
    (8, 2, 200, 16, 21, 256, 7),     # G = 4: more steps than the window holds
    (28, 4, 300, 8, 10, 320, 5),     # G = 7 (Qwen-like group)
    (4, 4, 97, 1, 4, 101, 2),        # G = 1, window of one row, ragged n
    (16, 2, 1030, 40, 3, 1100, 3),   # G = 8, n across the 1024-token workgroup edge
    (8, 2, 600, 130, 3, 640, 3),     # G = 4, w = 130: the window takes five 128-row launches, the last ragged
])
def test_decode_matches_oracle(Hq, Hkv, n0, w, steps, n_max, check_every):
    sc, q_all, k, v, kc, vc = _setup(Hq, Hkv, n0, w, steps, n_max)
    S0 = sc.raw_scores().cpu().numpy()
    sc.check()
    err = max_rel_err(S0, _ref(q_all, k, v, n0, w, Hq, Hkv))
    assert err <= RTOL["bf16"], f"after init: {err}"
    for s in range(steps):
        sc.step(_dev(q_all[:, n0 + s]).contiguous(), kc, vc)
        if (s + 1) % check_every == 0 or s + 1 == steps:
            n = n0 + s + 1
            S = sc.raw_scores().cpu().numpy()
            sc.check()
            err = max_rel_err(S, _ref(q_all, k, v, n, w, Hq, Hkv))
            assert err <= RTOL["bf16"], f"after {s + 1} steps: {err}"
    S64 = sc.raw_scores_f64().cpu().numpy()
    S32 = sc.raw_scores().cpu().numpy()
    np.testing.assert_array_equal(S32, S64.astype(np.float32))


@pytest.mark.parametrize("Hq,Hkv,n0,w,steps", [(8, 2, 300, 12, 30), (28, 4, 200, 6, 9)])
def test_incremental_equals_rebuild(Hq, Hkv, n0, w, steps):
    sc, q_all, k, v, kc, vc = _setup(Hq, Hkv, n0, w, steps, n0 + steps + 5, needles=8)
    for s in range(steps):
        sc.step(_dev(q_all[:, n0 + s]).contiguous(), kc, vc)
    inc = sc.raw_scores_f64().cpu().numpy().copy()
    sc.rebuild(kc, vc)
    reb = sc.raw_scores_f64().cpu().numpy()
    sc.check()
    scale = np.abs(reb).max()
    assert scale > 0
    # terms of departed rows cancel exactly; what remains is fp64 summation order
    assert np.abs(inc - reb).max() <= 1e-12 * scale
    big = np.abs(reb) > 1e-6 * scale
    rel = np.abs(inc[big] - reb[big]) / np.abs(reb[big])
    assert rel.max() <= 1e-9, rel.max()


def test_reevict_matches_select_and_oracle():
    Hq, Hkv, n0, w, steps = 8, 2, 400, 16, 20
    sc, q_all, k, v, kc, vc = _setup(Hq, Hkv, n0, w, steps, 512, needles=6)
    for s in range(steps):
        sc.step(_dev(q_all[:, n0 + s]).contiguous(), kc, vc)
    n = n0 + steps
    ne = n - w - 37
    scores, idx = sc.select(pool_kernel=7, n_evict=ne)
    sc.check()
    raw = sc.raw_scores()
    s2, i2 = K.select(raw, window=w, pool_kernel=7, n_evict=ne)
    np.testing.assert_array_equal(scores.cpu().numpy(), s2.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), i2.cpu().numpy())
    ref = oracle.dropkv_oracle(q_all[:, n - w:n], k[:, :n], v[:, :n], n=n, window=w, Hq=Hq, Hkv=Hkv, d=128,
                               pool_kernel=7, n_evict=ne, dtype="bf16")
    assert max_rel_err(scores.cpu().numpy(), ref["P"]) <= RTOL["bf16"]
    exact, jac = check_evictions(scores.cpu().numpy(), idx.cpu().numpy(), ref["P"], ref["S"], ref["evict"], ne,
                                 RTOL["bf16"])
    print(f"exact heads {exact}/{Hkv}, jaccard {jac}")


def test_decode_rejects_invalid_calls():
    Hq, Hkv, w = 8, 2, 4
    with pytest.raises(K.DropKVInvalidError):
        K.DecodeScorer(n_max=64, window=w, Hq=Hq, Hkv=Hkv, d=64)
    sc, q_all, k, v, kc, vc = _setup(Hq, Hkv, 40, w, 1, 41)
    sc.step(_dev(q_all[:, 40]).contiguous(), kc, vc)  # fills the cache: n == n_max
    with pytest.raises(K.DropKVInvalidError):
        sc.step(_dev(q_all[:, 40]).contiguous(), kc, vc)  # n would exceed n_max
    lib = K.load_library()
    # init needs window < n; a step needs n >= window + 2; a small state is rejected
    q = _dev(q_all[:, 36:40]).contiguous()
    assert lib.dropkv_decode_init(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), w, 41, w, Hq, Hkv, 128,
                                  sc.state.data_ptr(), sc.state.numel(), sc.status.data_ptr(), None) == K.binding.ERR_INVALID
    assert lib.dropkv_decode_step(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), w + 1, 41, w, Hq, Hkv, 128,
                                  sc.state.data_ptr(), sc.state.numel(), sc.status.data_ptr(), None) == K.binding.ERR_INVALID
    assert lib.dropkv_decode_init(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), 40, 41, w, Hq, Hkv, 128,
                                  sc.state.data_ptr(), 1024, sc.status.data_ptr(), None) == K.binding.ERR_INVALID
    # a state in managed memory is refused (the single-pass step uses fp64 atomics on it)
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    ptr = ctypes.c_void_p()
    nbytes = sc.state.numel()
    assert hip.hipMallocManaged(ctypes.byref(ptr), ctypes.c_size_t(nbytes), ctypes.c_uint(1)) == 0
    try:
        assert lib.dropkv_decode_init(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), 40, 41, w, Hq, Hkv, 128,
                                      ptr.value, nbytes, sc.status.data_ptr(), None) == K.binding.ERR_INVALID
    finally:
        hip.hipFree(ptr)


def test_decode_reports_singular_new_row():
    Hq, Hkv, n0, w = 8, 2, 64, 4
    sc, q_all, k, v, kc, vc = _setup(Hq, Hkv, n0, w, 1, 80, needles=0)
    sc.check()
    qn = q_all[:, n0].copy()
    qf = synth.bf16_bits_to_float32(qn[1]).astype(np.float64)
    planted = (200.0 * qf / np.linalg.norm(qf)).astype(np.float32)
    kc[0, 9] = _dev(synth.bf16_round_bits(planted))  # query head 1's logit gap is ~200: rest mass << 2^-24
    sc.step(_dev(qn).contiguous(), kc, vc)
    with pytest.raises(K.DropKVSingularError):
        sc.check()


@pytest.mark.parametrize("workload,deferred", [("llama_128k", False), ("llama_128k", True),
                                               ("qwen_128k_sweep", True)])
def test_decode_full_layer_sampled(workload, deferred):
    """A 128K layer reached by decode steps, sized as the benchmark runs them:
    scored at n - 64 with 64 other window rows, then 64 appended positions whose
    query rows are the layer's window rows. The kept score is then the layer's
    score: against the oracle on sampled tokens (sink, needles, chunk edges,
    window edge, random), and against the scoring pass on every token. The
    Qwen-shaped layer (G = 7) takes the single-pass kernel for five to eight
    rows per position."""
    cfg = synth.CONFIGS[workload]
    case = synth.make_case(cfg)
    n, w, Hq, Hkv, d = case.n, case.window, case.Hq, case.Hkv, case.d
    q, k, v = to_torch(case)
    rng = np.random.default_rng(77)
    scale = float(synth.bf16_bits_to_float32(case.q).std())
    first = synth.bf16_round_bits((rng.standard_normal((Hq, w, d)) * scale).astype(np.float32))
    print(f"[decode full] {workload} n={n} w={w}: init at n - {w}, {w} steps, deferred={deferred}", flush=True)
    sc = K.DecodeScorer(n_max=n, window=w, Hq=Hq, Hkv=Hkv, d=d)
    sc.init(_dev(first).contiguous(), k, v, n - w)
    for i in range(w):
        sc.step(q[:, i].contiguous(), k, v, deferred=deferred)
    ne = cfg.n_evicts()[0]
    P, idx = sc.select(pool_kernel=cfg.pool_kernel, n_evict=ne)
    sc.check()
    S = sc.raw_scores().cpu().numpy()
    P, idx = P.cpu().numpy(), idx.cpu().numpy()
    for g in (0, Hkv - 1):
        e_S, e_P = check_sampled(case, g, cfg.pool_kernel, S, P, rng)
        print(f"[decode full] head {g}: sampled rel err S {e_S:.2e}, P {e_P:.2e}", flush=True)
    S_main = K.raw_scores(q, k, v).cpu().numpy()
    # each is within RTOL of the exact score
    assert max_rel_err(S, S_main) <= 2 * RTOL["bf16"]
    assert np.all(np.isinf(P[:, n - w:])) and np.all(np.isfinite(P[:, : n - w]))
    for g in range(Hkv):
        assert np.array_equal(idx[g], own_bottom_k(P[g], ne)), f"head {g}: not its own bottom-k"
    P_main, idx_main = K.select(torch.from_numpy(S_main).cuda(), window=w, pool_kernel=cfg.pool_kernel,
                                n_evict=ne)
    idx_main = idx_main.cpu().numpy()
    for g in range(Hkv):
        inter = np.intersect1d(idx[g], idx_main[g]).size
        jac = inter / (2 * ne - inter)
        assert jac > 0.99, f"head {g}: evicted set overlap with the scoring pass {jac:.4f}"


def _scorers(Hq, Hkv, n0, w, steps, n_max, needles=4):
    """Two scorers on the same grown cache, both initialised at n0."""
    a, q_all, k, v, kc, vc = _setup(Hq, Hkv, n0, w, steps, n_max, needles=needles)
    b = K.DecodeScorer(n_max=n_max, window=w, Hq=Hq, Hkv=Hkv, d=128)
    b.init(_dev(q_all[:, n0 - w:n0]).contiguous(), kc, vc, n0)
    return a, b, q_all, k, v, kc, vc


def _close_f64(x, y, rel):
    x, y = x.raw_scores_f64().cpu().numpy(), y.raw_scores_f64().cpu().numpy()
    scale = np.abs(y).max()
    assert scale > 0
    err = np.abs(x - y).max() / scale
    assert err <= rel, err
    return err


@pytest.mark.parametrize("Hq,Hkv,n0,w,steps,n_max", [
    (8, 2, 300, 12, 20, 330),     # G = 4, more steps than the window holds
    (28, 4, 2100, 6, 9, 2200),    # G = 7, two statistics chunks and a ragged tile
    (4, 4, 97, 1, 5, 110),        # G = 1, window of one row: the pending row is the one leaving
    (16, 2, 130, 20, 4, 140),     # G = 8, the largest group of the single pass
    (6, 2, 150, 7, 5, 160),       # G = 3
    (4, 2, 120, 3, 4, 130),       # G = 2
    (8, 2, 600, 130, 4, 640),     # G = 4 with a long window (rows leave from five init launches)
    (16, 1, 90, 5, 3, 100),       # G = 16: the deferred call takes the two-pass step
])
def test_deferred_steps_match_two_pass(Hq, Hkv, n0, w, steps, n_max):
    a, b, q_all, k, v, kc, vc = _scorers(Hq, Hkv, n0, w, steps, n_max)
    for s in range(steps):
        qn = _dev(q_all[:, n0 + s]).contiguous()
        a.step(qn, kc, vc, deferred=True)
        b.step(qn, kc, vc)
    a.check(), b.check()
    n = n0 + steps
    # the new rows' statistics take the same arithmetic in both forms; the terms too
    err = _close_f64(a, b, 1e-9)
    print(f"deferred vs two-pass: {err:.2e}")
    assert max_rel_err(a.raw_scores().cpu().numpy(), _ref(q_all, k, v, n, w, Hq, Hkv)) <= RTOL["bf16"]
    assert int(a.status.item()) & K.binding.STATUS_PENDING == 0


def test_deferred_mixed_with_two_pass_flush_and_rebuild():
    Hq, Hkv, n0, w, steps = 8, 2, 260, 10, 24
    a, b, q_all, k, v, kc, vc = _scorers(Hq, Hkv, n0, w, steps, 300, needles=6)
    plan = "DDTDFDDRTDDDTTDFFDDRDDTD"  # D deferred, T two-pass, F flush after a deferred step, R rebuild
    assert len(plan) == steps
    for s, op in enumerate(plan):
        qn = _dev(q_all[:, n0 + s]).contiguous()
        a.step(qn, kc, vc, deferred=op in "DFR")
        if op == "F":
            a.flush()
            a.flush()  # nothing left: a no-op
        if op == "R":
            a.rebuild(kc, vc)
        b.step(qn, kc, vc)
        if s % 6 == 5:
            a.check()
            n = n0 + s + 1
            assert max_rel_err(a.raw_scores().cpu().numpy(), _ref(q_all, k, v, n, w, Hq, Hkv)) <= RTOL["bf16"]
            _close_f64(a, b, 1e-9)
    a.check(), b.check()
    _close_f64(a, b, 1e-9)
    a.rebuild(kc, vc)
    _close_f64(a, b, 1e-9)


def test_select_reports_pending_terms():
    """The C entry points: select on a state with pending terms flags it; a flush clears it."""
    Hq, Hkv, n0, w = 8, 2, 200, 8
    sc, q_all, k, v, kc, vc = _setup(Hq, Hkv, n0, w, 2, 210)
    lib = K.load_library()
    args = (sc.n_max, w, Hq, Hkv, 128)
    stream = torch.cuda.current_stream().cuda_stream
    qn = _dev(q_all[:, n0]).contiguous()
    assert lib.dropkv_decode_step_deferred(qn.data_ptr(), kc.data_ptr(), vc.data_ptr(), n0 + 1, *args,
                                           sc.state.data_ptr(), sc.state.numel(), sc.status.data_ptr(), stream) == 0
    n = n0 + 1
    out = torch.empty((Hkv, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((Hkv, 10), dtype=torch.int64, device="cuda")
    assert lib.dropkv_decode_select(sc.state.data_ptr(), sc.state.numel(), n, *args, 3, 10, out.data_ptr(),
                                    idx.data_ptr(), sc.status.data_ptr(), stream) == 0
    assert int(sc.status.item()) == K.binding.STATUS_PENDING
    partial = out.clone()
    sc.status.zero_()
    assert lib.dropkv_decode_flush(kc.data_ptr(), vc.data_ptr(), n, *args, sc.state.data_ptr(), sc.state.numel(),
                                   stream) == 0
    assert lib.dropkv_decode_select(sc.state.data_ptr(), sc.state.numel(), n, *args, 3, 10, out.data_ptr(),
                                    idx.data_ptr(), sc.status.data_ptr(), stream) == 0
    assert int(sc.status.item()) == 0
    ref = oracle.dropkv_oracle(q_all[:, n - w:n], k[:, :n], v[:, :n], n=n, window=w, Hq=Hq, Hkv=Hkv, d=128,
                               pool_kernel=3, n_evict=10, dtype="bf16")
    assert max_rel_err(out.cpu().numpy(), ref["P"]) <= RTOL["bf16"]
    # before the flush the newest position's terms were missing
    assert max_rel_err(partial.cpu().numpy(), ref["P"]) > RTOL["bf16"]
