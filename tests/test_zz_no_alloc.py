"""dropkv_score_noalloc (scratch in the library's static device array) against
dropkv_score_ex (scratch in a caller workspace), through the C ABI.

Both run the same kernels, so scores and evicted sets must agree bit for bit.
Two calls in a row on one GPU, the second on a smaller input (the array keeps
the first call's contents, so anything the second call failed to clear would
show), on the MFMA path and on the plain-VALU path; then a shape whose
workspace exceeds the array is rejected before anything is launched.
"""

import ctypes

import numpy as np
import pytest

import kv_cache_eviction_pass1_amd as K
from kv_cache_eviction_pass1_amd import binding, synth
from parity import to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    yield


def _both(case, pool, ne):
    q, k, v = to_torch(case)
    dcode = K.BF16 if case.dtype == "bf16" else K.F32
    ws = torch.empty(K.workspace_bytes(dcode, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device="cuda")
    st_ex = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    sc_ex, ix_ex = K.score_ex(q, k, v, pool_kernel=pool, n_evict=ne, workspace=ws, status=st_ex)
    st_na = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    sc_na = torch.full((case.Hkv, case.n), -7.0, dtype=torch.float32, device="cuda")
    ix_na = torch.full((case.Hkv, ne), -7, dtype=torch.int64, device="cuda")
    binding.score_noalloc(q, k, v, pool_kernel=pool, n_evict=ne, status=st_na, scores=sc_na, evict_idx=ix_na)
    torch.cuda.synchronize()
    assert int(st_ex.item()) == 0 and int(st_na.item()) == 0
    a, b = sc_ex.cpu().numpy(), sc_na.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "scores differ"
    assert np.array_equal(ix_ex.cpu().numpy(), ix_na.cpu().numpy()), "evicted sets differ"


@pytest.mark.parametrize("big,small", [("llama_32k", "llama_4k")])
def test_noalloc_matches_ex_two_calls_mfma(big, small):
    for name in (big, small):
        cfg = synth.CONFIGS[name]
        case = synth.make_case(cfg)
        print(f"[noalloc] {name} n={case.n}", flush=True)
        _both(case, cfg.pool_kernel, cfg.n_evicts()[0])


def test_noalloc_matches_ex_two_calls_generic():
    for n, w, ne in ((3000, 17, 1200), (257, 5, 40)):
        case = synth.make_gaussian_case(Hq=8, Hkv=2, d=64, n=n, window=w, dtype="f32", seeds=(n, n + 1, n + 2))
        print(f"[noalloc] f32 n={n}", flush=True)
        _both(case, 5, ne)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    lib = K.load_library()
    q = torch.zeros((32, 64, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((8, 64, 128), dtype=torch.bfloat16, device="cuda")
    sc = torch.zeros((8, 64), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_big = 1 << 20  # claimed token count: its workspace exceeds the array; nothing may be launched
    assert K.workspace_bytes(K.BF16, n_big, 64, 32, 8, 128) > binding.NOALLOC_SCRATCH_BYTES
    rc = lib.dropkv_score_noalloc(K.BF16, q.data_ptr(), kv.data_ptr(), kv.data_ptr(), n_big, 64, 32, 8, 128,
                                  7, 0, sc.data_ptr(), None, st.data_ptr(), 0, None)
    assert rc == binding.ERR_INVALID
    assert b"SCRATCH" in lib.dropkv_last_error()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    # the 128K Llama layer fits
    assert K.workspace_bytes(K.BF16, 131072, 64, 32, 8, 128) <= binding.NOALLOC_SCRATCH_BYTES
