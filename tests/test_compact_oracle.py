"""Pins of the cache-compaction oracle (CPU).

The oracle selects kept rows with a boolean mask; these tests check it against
a walk that merges the token range with the sorted eviction list (a different
algorithm), against the identities of the operation (nothing evicted, all
evicted, kept plus evicted = every token once, in order), and on its error
cases.
"""

import numpy as np
import pytest

import oracle


def _walk(k, v, evict):
    """Two-pointer merge of 0..n-1 with the eviction list: the kept rows in order."""
    n_keep = k.shape[1] - evict.shape[1]
    out_k = np.empty((k.shape[0], n_keep) + k.shape[2:], k.dtype)
    out_v = np.empty((v.shape[0], n_keep) + v.shape[2:], v.dtype)
    for g in range(k.shape[0]):
        e = list(evict[g])
        i, r = 0, 0
        for j in range(k.shape[1]):
            if i < len(e) and e[i] == j:
                i += 1
                continue
            out_k[g, r] = k[g, j]
            out_v[g, r] = v[g, j]
            r += 1
        assert r == n_keep
    return out_k, out_v


@pytest.mark.parametrize("Hkv,n,d,ne,seed", [(1, 1, 1, 0, 0), (2, 9, 3, 4, 1), (3, 50, 8, 49, 2),
                                             (2, 300, 5, 120, 3), (1, 17, 2, 17, 4)])
def test_compaction_matches_merge_walk(Hkv, n, d, ne, seed):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 1 << 16, size=(Hkv, n, d)).astype(np.uint16)  # bf16 bit patterns
    v = rng.standard_normal((Hkv, n, d)).astype(np.float32)
    evict = np.stack([np.sort(rng.choice(n, size=ne, replace=False)) for _ in range(Hkv)]).astype(np.int64)
    ok, ov = oracle.compact_cache(k, v, evict)
    wk, wv = _walk(k, v, evict)
    assert ok.shape == (Hkv, n - ne, d) and ok.dtype == k.dtype
    assert np.array_equal(ok, wk) and np.array_equal(ov.view(np.uint32), wv.view(np.uint32))


def test_compaction_identities():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((2, 40, 4)).astype(np.float32)
    v = rng.standard_normal((2, 40, 4)).astype(np.float32)
    ok, ov = oracle.compact_cache(k, v, np.zeros((2, 0), np.int64))
    assert np.array_equal(ok, k) and np.array_equal(ov, v)
    ok, ov = oracle.compact_cache(k, v, np.tile(np.arange(40), (2, 1)))
    assert ok.shape == (2, 0, 4) and ov.shape == (2, 0, 4)
    # kept rows plus evicted rows are every row once: tag rows with their index
    tag = np.tile(np.arange(40, dtype=np.float32)[None, :, None], (2, 1, 4))
    evict = np.array([[0, 5, 6, 39], [1, 2, 3, 20]], np.int64)
    ok, _ = oracle.compact_cache(tag, tag, evict)
    for g in range(2):
        kept = ok[g, :, 0].astype(int)
        assert np.all(np.diff(kept) > 0)
        assert sorted(kept.tolist() + evict[g].tolist()) == list(range(40))


@pytest.mark.parametrize("bad", [[3, 3], [5, 2], [-1, 4], [0, 40]])
def test_compaction_rejects_bad_lists(bad):
    k = np.zeros((1, 40, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.compact_cache(k, k, np.array([bad], np.int64))
