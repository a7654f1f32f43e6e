"""Exact invariances of the score on the GPU, through the C ABI.

Doubling every value vector doubles a (a = sum p_j v_j, and bf16 rounding
commutes with a power-of-two scale), leaves every p untouched (it depends on
q and k only) and so multiplies every term r^2 ||a - v_j||^2, the argmax
terms and the rest by exactly 4: every fp32 and fp64 operation on the path
sees operands scaled by powers of two, which round the same way. The raw and
pooled scores must therefore come out multiplied by 4 bit for bit and the
evicted sets must not change, on the MFMA path, the plain-VALU path and the
decode-time rescoring. A dropped or doubled term, a mixed-up operand (q for
a, k for v) or a tolerance-hidden drift in the value path breaks this.
"""

import dataclasses

import numpy as np
import pytest

import kv_cache_eviction_pass1_amd as K
from kv_cache_eviction_pass1_amd import synth
from parity import to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    yield


def _doubled_v(case):
    if case.dtype == "bf16":
        v2 = synth.bf16_round_bits(2.0 * synth.bf16_bits_to_float32(case.v))  # exact: a power of two
        assert np.array_equal(synth.bf16_bits_to_float32(v2), 2.0 * synth.bf16_bits_to_float32(case.v))
    else:
        v2 = (2.0 * case.v).astype(np.float32)
    return dataclasses.replace(case, v=v2)


@pytest.mark.parametrize("workload,n,dtype", [
    ("llama_4k", 4096, "bf16"),     # MFMA path: pass 1, merge, fix-up, pass 2, select
    ("llama_4k", 1500, "bf16"),     # ragged n
    ("tiny", 300, "f32"),           # plain-VALU path
])
def test_doubling_values_quadruples_scores(workload, n, dtype):
    cfg = synth.CONFIGS[workload]
    case = synth.make_case(cfg, n=n, dtype=dtype)
    case2 = _doubled_v(case)
    ne = (n - case.window) // 2
    outs = []
    for c in (case, case2):
        q, k, v = to_torch(c)
        S = K.raw_scores(q, k, v).cpu().numpy()
        P, idx = K.score(q, k, v, pool_kernel=cfg.pool_kernel, n_evict=ne)
        outs.append((S, P.cpu().numpy(), idx.cpu().numpy()))
    (S1, P1, i1), (S2, P2, i2) = outs
    assert np.any(S1 > 0)
    np.testing.assert_array_equal(S2, 4.0 * S1)
    np.testing.assert_array_equal(P2, 4.0 * P1)  # +inf stays +inf
    np.testing.assert_array_equal(i2, i1)


@pytest.mark.parametrize("deferred", [False, True])
def test_doubling_values_quadruples_decode_scores(deferred):
    Hq, Hkv, d, n0, w, steps = 8, 2, 128, 260, 9, 12
    q_all, k, v = synth.make_decode_case(Hq, Hkv, d, n0 + steps, needles=4)
    v2 = synth.bf16_round_bits(2.0 * synth.bf16_bits_to_float32(v))
    dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16).copy()).view(torch.bfloat16).cuda()
    res = []
    for vv in (v, v2):
        kc, vc = dev(k), dev(vv)
        sc = K.DecodeScorer(n_max=n0 + steps, window=w, Hq=Hq, Hkv=Hkv, d=d)
        sc.init(dev(q_all[:, n0 - w:n0]).contiguous(), kc, vc, n0)
        for s in range(steps):
            sc.step(dev(q_all[:, n0 + s]).contiguous(), kc, vc, deferred=deferred)
        S64 = sc.raw_scores_f64().cpu().numpy().copy()
        P, idx = sc.select(pool_kernel=5, n_evict=100)
        sc.check()
        res.append((S64, P.cpu().numpy(), idx.cpu().numpy()))
    (S1, P1, i1), (S2, P2, i2) = res
    assert np.any(S1 > 0)
    np.testing.assert_array_equal(S2, 4.0 * S1)
    np.testing.assert_array_equal(P2, 4.0 * P1)
    np.testing.assert_array_equal(i2, i1)


@pytest.mark.parametrize("workload,n,dtype", [("llama_4k", 2500, "bf16"), ("tiny", 300, "f32")])
def test_reversing_kv_heads_reverses_outputs(workload, n, dtype):
    """Each KV head's score depends only on its own K/V and query group: listing
    the heads (with their groups) in reverse order must reverse the outputs bit
    for bit. A head-stride or group-offset mistake breaks this."""
    cfg = synth.CONFIGS[workload]
    case = synth.make_case(cfg, n=n, dtype=dtype)
    G = case.Hq // case.Hkv
    qr = case.q.reshape(case.Hkv, G, *case.q.shape[1:])[::-1].reshape(case.q.shape)
    rev = dataclasses.replace(case, q=np.ascontiguousarray(qr), k=np.ascontiguousarray(case.k[::-1]),
                              v=np.ascontiguousarray(case.v[::-1]))
    ne = (n - case.window) // 3
    outs = []
    for c in (case, rev):
        q, k, v = to_torch(c)
        S = K.raw_scores(q, k, v).cpu().numpy()
        P, idx = K.score(q, k, v, pool_kernel=cfg.pool_kernel, n_evict=ne)
        outs.append((S, P.cpu().numpy(), idx.cpu().numpy()))
    (S1, P1, i1), (S2, P2, i2) = outs
    np.testing.assert_array_equal(S2, S1[::-1])
    np.testing.assert_array_equal(P2, P1[::-1])
    np.testing.assert_array_equal(i2, i1[::-1])
