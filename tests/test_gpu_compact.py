"""Cache compaction on the GPU (dropkv_compact) against the oracle, bit for bit.

Covers the three copy widths (16-, 4- and 2-byte units, chosen from the row
size and the pointers' alignment), ragged row counts around the 128-row
output block, empty and full eviction lists, kept sets of every shape (spread
out, in runs, all at the front, all at the back, at both ends around one long
evicted run: the case whose block span holds more list entries than the
kernel stages in LDS), invalid lists (status bit, and no write outside the
outputs: guard rows around them stay untouched), and the score -> compact
pipeline on a full-size layer. The kept-list form (dropkv_compact_kept, fed
by the kept list dropkv_score_keep_ex writes) is checked the same way: against
the oracle's compaction of the complementary eviction list, on invalid lists,
and score -> compact on the 32K layer.
"""

import numpy as np
import pytest

import oracle
import kv_cache_eviction_pass1_amd as K
from kv_cache_eviction_pass1_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GUARD = 3  # guard rows on each side of every output


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    yield


def _bits(t):
    """Host copy of a tensor's bit patterns."""
    a = t.detach().cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy()
    return a.view(torch.int32).numpy()


def _guarded_outputs(Hkv, n_keep, d, dtype, dev):
    """Outputs as views into larger buffers whose guard rows hold a fill pattern."""
    bufs, views = [], []
    for _ in range(2):
        b = torch.full((Hkv * n_keep * d + 2 * GUARD * d,), -7.0, dtype=dtype, device=dev)
        bufs.append(b)
        views.append(b[GUARD * d: GUARD * d + Hkv * n_keep * d].view(Hkv, n_keep, d))
    return bufs, views


def _check_guards(bufs, Hkv, n_keep, d):
    for b in bufs:
        head = b[: GUARD * d].float().cpu()
        tail = b[GUARD * d + Hkv * n_keep * d:].float().cpu()
        assert torch.all(head == -7.0) and torch.all(tail == -7.0), "write outside the output"


def _evict_lists(rng, Hkv, n, ne, kind):
    rows = []
    for g in range(Hkv):
        if kind == "random":
            e = np.sort(rng.choice(n, size=ne, replace=False))
        elif kind == "runs":  # long runs of kept and evicted tokens
            starts = np.sort(rng.choice(max(n - 1, 1), size=max(1, ne // 50), replace=False))
            e = np.unique(np.concatenate([np.arange(s, min(n, s + 50)) for s in starts]))[:ne]
            if e.size < ne:
                rest = np.setdiff1d(np.arange(n), e)
                e = np.sort(np.concatenate([e, rng.choice(rest, size=ne - e.size, replace=False)]))
        elif kind == "front":  # keep the first tokens
            e = np.arange(n - ne, n)
        elif kind == "back":  # keep the last tokens
            e = np.arange(0, ne)
        elif kind == "ends":  # keep both ends, one evicted run between them
            s0 = (n - ne) // 2
            e = np.arange(s0, s0 + ne)
        else:  # every other token, from g
            e = np.arange(g % 2, n, 2)[:ne]
            if e.size < ne:
                rest = np.setdiff1d(np.arange(n), e)
                e = np.sort(np.concatenate([e, rest[: ne - e.size]]))
        rows.append(e.astype(np.int64))
    return np.stack(rows) if rows else np.zeros((Hkv, 0), np.int64)


def _run(k, v, ev, misalign=False):
    Hkv, n, d = k.shape
    n_keep = n - ev.shape[1]
    bufs, (ok, ov) = _guarded_outputs(Hkv, n_keep, d, k.dtype, k.device)
    if misalign:  # inputs one element past an aligned base: forces the 2-byte / 4-byte copy
        kb = torch.empty(k.numel() + 1, dtype=k.dtype, device=k.device)
        vb = torch.empty(v.numel() + 1, dtype=v.dtype, device=v.device)
        kb[1:].copy_(k.reshape(-1))
        vb[1:].copy_(v.reshape(-1))
        k, v = kb[1:].view(Hkv, n, d), vb[1:].view(Hkv, n, d)
    st = torch.zeros(1, dtype=torch.int32, device=k.device)
    K.compact(k, v, torch.from_numpy(ev).to(k.device), status=st, out_k=ok, out_v=ov)
    torch.cuda.synchronize()
    return ok, ov, int(st.item()), bufs


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 7), ("f32", 3), ("f32", 64), ("bf16", 256)])
@pytest.mark.parametrize("n", [1, 5, 1025, 3000, 4095, 4096, 4097, 9000])
def test_compact_matches_oracle(dtype, d, n):
    rng = np.random.default_rng(n * 31 + d)
    Hkv = 3
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.randn(Hkv, n, d).to(tdt).cuda()
    v = torch.randn(Hkv, n, d).to(tdt).cuda()
    for ne, kind in ((0, "random"), (n, "random"), (n // 2, "random"), (n - n // 7, "runs"), (n // 3, "alt"),
                     (n - n // 7, "front"), (n // 2, "back"), (n - n // 7, "ends")):
        ev = _evict_lists(rng, Hkv, n, ne, kind)
        print(f"[compact] {dtype} d={d} n={n} evict={ne} {kind}", flush=True)
        ok, ov, st, bufs = _run(k, v, ev)
        assert st == 0
        rk, rv = oracle.compact_cache(_bits(k), _bits(v), ev)
        assert np.array_equal(_bits(ok), rk) and np.array_equal(_bits(ov), rv)
        _check_guards(bufs, Hkv, n - ne, d)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 32)])
def test_compact_unaligned_inputs(dtype, d):
    rng = np.random.default_rng(5)
    Hkv, n = 2, 2500
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.randn(Hkv, n, d).to(tdt).cuda()
    v = torch.randn(Hkv, n, d).to(tdt).cuda()
    ev = _evict_lists(rng, Hkv, n, 1900, "random")
    print(f"[compact] unaligned {dtype} d={d}", flush=True)
    ok, ov, st, bufs = _run(k, v, ev, misalign=True)
    assert st == 0
    rk, rv = oracle.compact_cache(_bits(k), _bits(v), ev)
    assert np.array_equal(_bits(ok), rk) and np.array_equal(_bits(ov), rv)
    _check_guards(bufs, Hkv, n - 1900, d)


@pytest.mark.parametrize("bad", ["unsorted", "duplicate", "too_large", "negative"])
def test_compact_bad_lists_flagged_and_contained(bad):
    Hkv, n, d = 2, 3000, 16
    k = torch.randn(Hkv, n, d).cuda()
    v = torch.randn(Hkv, n, d).cuda()
    rng = np.random.default_rng(9)
    ev = _evict_lists(rng, Hkv, n, 1000, "random")
    if bad == "unsorted":
        ev[1, 10], ev[1, 500] = ev[1, 500], ev[1, 10]
    elif bad == "duplicate":
        ev[0, 700] = ev[0, 699]
    elif bad == "too_large":
        ev[1, -1] = n + 5
    else:
        ev[0, 0] = -3
    print(f"[compact] bad list: {bad}", flush=True)
    ok, ov, st, bufs = _run(k, v, ev)
    assert st & K.STATUS_BAD_INDEX
    _check_guards(bufs, Hkv, n - 1000, d)
    with pytest.raises(K.DropKVInvalidError):
        K.compact(k, v, torch.from_numpy(ev).cuda())


def test_compact_invalid_arguments_launch_nothing():
    k = torch.randn(2, 100, 8).cuda()
    ev = torch.zeros((2, 101), dtype=torch.int64, device="cuda")
    with pytest.raises(K.DropKVInvalidError):
        K.compact(k, k.clone(), ev)  # more evictions than tokens
    with pytest.raises(K.DropKVInvalidError):
        K.compact(k, k.clone(), torch.zeros((3, 4), dtype=torch.int64, device="cuda"))


def test_score_then_compact_full_layer():
    """The step after scoring: the 32K Llama layer, scored, then its cache compacted."""
    cfg = synth.CONFIGS["llama_32k"]
    case = synth.make_case(cfg)
    to_t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = to_t(case.q), to_t(case.k), to_t(case.v)
    ne = cfg.n_evicts()[0]
    print(f"[compact] score -> compact llama_32k evict={ne}", flush=True)
    _, idx = K.score(q, k, v, pool_kernel=cfg.pool_kernel, n_evict=ne)
    ok, ov = K.compact(k, v, idx)
    torch.cuda.synchronize()
    rk, rv = oracle.compact_cache(case.k, case.v, idx.cpu().numpy())
    assert ok.shape == (case.Hkv, case.n - ne, case.d)
    assert np.array_equal(_bits(ok), rk.view(np.int16)) and np.array_equal(_bits(ov), rv.view(np.int16))
    # the protected window is always kept, at the end of every head
    assert np.array_equal(_bits(ok)[:, -case.window:], case.k[:, -case.window:].view(np.int16))


def _keep_lists(ev, n):
    """Per head the token indices an eviction list does not name, ascending."""
    return np.stack([np.setdiff1d(np.arange(n), e) for e in ev]).astype(np.int64) if len(ev) else \
        np.zeros((0, n), np.int64)


def _run_kept(k, v, keep):
    Hkv, n, d = k.shape
    n_keep = keep.shape[1]
    bufs, (ok, ov) = _guarded_outputs(Hkv, n_keep, d, k.dtype, k.device)
    st = torch.zeros(1, dtype=torch.int32, device=k.device)
    K.compact_kept(k, v, torch.from_numpy(np.ascontiguousarray(keep)).to(k.device), status=st, out_k=ok, out_v=ov)
    torch.cuda.synchronize()
    return ok, ov, int(st.item()), bufs


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 7), ("f32", 3)])
@pytest.mark.parametrize("n", [1, 1025, 4097, 9000])
def test_compact_kept_matches_oracle(dtype, d, n):
    """dropkv_compact_kept on the complement of each eviction list gives the
    oracle's compaction of that list, bit for bit."""
    rng = np.random.default_rng(n * 7 + d)
    Hkv = 3
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.randn(Hkv, n, d).to(tdt).cuda()
    v = torch.randn(Hkv, n, d).to(tdt).cuda()
    for ne, kind in ((0, "random"), (n, "random"), (n // 2, "random"), (n - n // 7, "runs"),
                     (n - n // 7, "front"), (n // 2, "back"), (n - n // 7, "ends")):
        ev = _evict_lists(rng, Hkv, n, ne, kind)
        keep = _keep_lists(ev, n)
        print(f"[compact_kept] {dtype} d={d} n={n} keep={n - ne} {kind}", flush=True)
        ok, ov, st, bufs = _run_kept(k, v, keep)
        assert st == 0
        rk, rv = oracle.compact_cache(_bits(k), _bits(v), ev)
        assert np.array_equal(_bits(ok), rk) and np.array_equal(_bits(ov), rv)
        _check_guards(bufs, Hkv, n - ne, d)


@pytest.mark.parametrize("bad", ["unsorted", "duplicate", "too_large", "negative"])
def test_compact_kept_bad_lists_flagged_and_contained(bad):
    Hkv, n, d = 2, 3000, 16
    k = torch.randn(Hkv, n, d).cuda()
    v = torch.randn(Hkv, n, d).cuda()
    keep = _keep_lists(_evict_lists(np.random.default_rng(4), Hkv, n, 1000, "random"), n)
    if bad == "unsorted":
        keep[1, 10], keep[1, 500] = keep[1, 500], keep[1, 10]
    elif bad == "duplicate":
        keep[0, 700] = keep[0, 699]
    elif bad == "too_large":
        keep[1, -1] = n + 5
    else:
        keep[0, 0] = -3
    print(f"[compact_kept] bad list: {bad}", flush=True)
    ok, ov, st, bufs = _run_kept(k, v, keep)
    assert st & K.STATUS_BAD_INDEX
    _check_guards(bufs, Hkv, keep.shape[1], d)
    with pytest.raises(K.DropKVInvalidError):
        K.compact_kept(k, v, torch.from_numpy(keep).cuda())


@pytest.mark.parametrize("n,w,Hq,Hkv,ne", [(3000, 16, 8, 2, 1500), (3000, 16, 8, 2, 0), (3000, 16, 8, 2, 2984),
                                          (65, 1, 4, 2, 30), (4161, 17, 6, 2, 4000)])
def test_score_keep_list_is_the_complement(n, w, Hq, Hkv, ne):
    """dropkv_score_keep_ex: the same scores and evicted sets as dropkv_score_ex,
    and per head a kept list that is exactly the complement, ascending."""
    case = synth.make_gaussian_case(Hq, Hkv, 128, n, w, dtype="bf16", seeds=(n, w, ne), sink=True, needles=8)
    to_t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = to_t(case.q), to_t(case.k), to_t(case.v)
    ws = torch.empty(K.workspace_bytes(K.BF16, n, w, Hq, Hkv, 128), dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"[score_keep] n={n} w={w} Hq={Hq} Hkv={Hkv} evict={ne}", flush=True)
    s0, i0 = K.score_ex(q, k, v, pool_kernel=7, n_evict=ne, workspace=ws, status=st)
    s1, i1, kp = K.score_keep_ex(q, k, v, pool_kernel=7, n_evict=ne, workspace=ws, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(s0, s1) and torch.equal(i0, i1)
    assert kp.shape == (Hkv, n - ne)
    assert np.array_equal(kp.cpu().numpy(), _keep_lists(i1.cpu().numpy(), n))


def test_score_keep_then_compact_kept_full_layer():
    """Score the 32K Llama layer with its kept list, then compact from it: the
    same cache as compaction from the eviction list."""
    cfg = synth.CONFIGS["llama_32k"]
    case = synth.make_case(cfg)
    to_t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = to_t(case.q), to_t(case.k), to_t(case.v)
    ne = cfg.n_evicts()[0]
    ws = torch.empty(K.workspace_bytes(K.BF16, case.n, case.window, case.Hq, case.Hkv, case.d),
                     dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"[compact_kept] score -> compact_kept llama_32k evict={ne}", flush=True)
    _, idx, keep = K.score_keep_ex(q, k, v, pool_kernel=cfg.pool_kernel, n_evict=ne, workspace=ws, status=st)
    ok1, ov1 = K.compact_kept(k, v, keep)
    ok0, ov0 = K.compact(k, v, idx)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(ok0, ok1) and torch.equal(ov0, ov1)
    assert np.array_equal(keep.cpu().numpy(), _keep_lists(idx.cpu().numpy(), case.n))
