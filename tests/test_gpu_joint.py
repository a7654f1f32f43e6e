"""The approximation-ratio diagnostic on the GPU's own eviction sets.

Tiny fp32 cases are scored through the C ABI; the joint objective of the
returned set is compared with the brute-force optimum (CPU, fp64). The GPU
set must match the oracle's DropKV set (then its cost is the oracle's) and
can never beat the optimum.
"""

import numpy as np
import pytest

import kv_cache_eviction_pass1_amd as K
from oracle.joint import approx_ratio, joint_objective

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    yield


@pytest.mark.parametrize("ne,pool", [(3, 1), (5, 1), (3, 3)])
def test_gpu_selection_ratio(ne, pool):
    Hq, Hkv, d, n, w = 4, 2, 8, 14, 3
    ratios = []
    for seed in range(6):
        rng = np.random.default_rng(300 + seed)
        q = rng.standard_normal((Hq, w, d)).astype(np.float32)
        k = (rng.standard_normal((Hkv, n, d)) * 1.5).astype(np.float32)
        v = rng.standard_normal((Hkv, n, d)).astype(np.float32)
        print(f"[joint] seed {300 + seed} evict {ne} pool {pool}", flush=True)
        _, idx = K.score(*(torch.from_numpy(t).cuda() for t in (q, k, v)), pool_kernel=pool, n_evict=ne)
        idx = idx.cpu().numpy()
        r = approx_ratio(q, k, v, n=n, window=w, Hq=Hq, Hkv=Hkv, d=d, n_evict=ne, pool_kernel=pool,
                         dtype="f32")
        for g in range(Hkv):
            J = joint_objective(q, k, v, g, Hq // Hkv, n, w, idx[g], dtype="f32")
            assert J >= r["J_opt"][g] * (1 - 1e-12)
            assert abs(J - r["J_dropkv"][g]) <= 1e-12 * r["J_dropkv"][g]
            ratios.append(J / r["J_opt"][g])
    print(f"[joint] GPU sets, evict {ne} pool {pool}: ratio median {np.median(ratios):.4f} "
          f"max {np.max(ratios):.4f}")
