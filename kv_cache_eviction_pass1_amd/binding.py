"""ctypes binding of libdropkv (argument marshalling only).

Every step of the scoring runs in the HIP library; this module only checks
tensor shapes, allocates outputs with torch on the inputs' device and passes
raw pointers and the current HIP stream. If the library is not built, or no
GPU is present, calls raise: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# DROPKV_LIBRARY may name one of the checking builds next to it
# (libdropkv_debug.so, libdropkv_asan.so; see build.py) instead.
LIB_PATH = os.environ.get("DROPKV_LIBRARY") or os.path.join(_HERE, "libdropkv.so")

OK, ERR_INVALID, ERR_SINGULAR, ERR_NONFINITE, ERR_DEVICE, ERR_NEGATIVE = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
STATUS_SINGULAR, STATUS_NONFINITE, STATUS_BAD_INDEX, STATUS_PENDING, STATUS_NEGATIVE = 1, 2, 4, 8, 16
FLAG_GENERIC = 1
FLAG_STAGE_LOG = 2

# name -> (restype, argtypes)
_c = ctypes
_p, _i32, _i64, _u32, _sz = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_uint32, _c.c_size_t
SIGNATURES = {
    "dropkv_score": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p, _p]),
    "dropkv_score_f32": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p, _p]),
    "dropkv_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "dropkv_score_ex": (_i32, [_i32, _p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p,
                               _p, _sz, _p, _u32, _p]),
    "dropkv_score_keep_ex": (_i32, [_i32, _p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p,
                                    _p, _p, _sz, _p, _u32, _p]),
    "dropkv_score_noalloc": (_i32, [_i32, _p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p,
                                    _p, _u32, _p]),
    "dropkv_raw_scores": (_i32, [_i32, _p, _p, _p, _i64, _i32, _i32, _i32, _i32, _p, _u32, _p]),
    "dropkv_row_stats": (_i32, [_i32, _p, _p, _p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p,
                                _u32, _p]),
    "dropkv_pass1_stats": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
    "dropkv_select": (_i32, [_p, _i64, _i32, _i32, _i32, _i64, _p, _p, _p]),
    "dropkv_stage_times": (_i32, [_i32, _p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p,
                                  _p, _u32, _p, _p, _i32, _p, _p]),
    "dropkv_stage_log": (_i32, [_p, _p, _i32, _p, _p]),
    "dropkv_score_from_stats": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p,
                                       _p, _p, _p, _p, _p]),
    "dropkv_score_from_stats_ex": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p,
                                          _p, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "dropkv_prefill_attention": (_i32, [_p, _p, _p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p,
                                        _p]),
    "dropkv_compact": (_i32, [_i32, _p, _p, _i64, _i32, _i32, _p, _i64, _p, _p, _p, _p]),
    "dropkv_compact_kept": (_i32, [_i32, _p, _p, _i64, _i32, _i32, _p, _i64, _p, _p, _p, _p]),
    "dropkv_decode_state_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "dropkv_decode_init": (_i32, [_p, _p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _sz, _p, _p]),
    "dropkv_decode_step": (_i32, [_p, _p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _sz, _p, _p]),
    "dropkv_decode_step_deferred": (_i32, [_p, _p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _sz, _p, _p]),
    "dropkv_decode_flush": (_i32, [_p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _sz, _p]),
    "dropkv_decode_rebuild": (_i32, [_p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _sz, _p, _p]),
    "dropkv_decode_scores": (_i32, [_p, _sz, _i64, _i64, _i32, _i32, _i32, _i32, _p, _p]),
    "dropkv_decode_select": (_i32, [_p, _sz, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _p, _p, _p,
                                    _p]),
    "dropkv_uses_mfma": (_i32, [_i32, _i32]),
    "dropkv_last_error": (_c.c_char_p, []),
    "dropkv_last_error_string": (_c.c_char_p, []),
    "dropkv_version": (_c.c_char_p, []),
}


class DropKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dropkv error {code}: {msg}")
        self.code = code


class DropKVInvalidError(DropKVError, ValueError):
    pass


class DropKVSingularError(DropKVError):
    pass


class DropKVNonFiniteError(DropKVError):
    pass


class DropKVNegativeScoreError(DropKVError, ValueError):
    pass


class DropKVNotBuiltError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdropkv.so (raises DropKVNotBuiltError if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise DropKVNotBuiltError(f"{path} is missing: build the HIP library first "
                                  "(python -m kv_cache_eviction_pass1_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _raise(code: int):
    if code == OK:
        return
    msg = load_library().dropkv_last_error().decode(errors="replace")
    cls = {ERR_INVALID: DropKVInvalidError, ERR_SINGULAR: DropKVSingularError,
           ERR_NONFINITE: DropKVNonFiniteError,
           ERR_NEGATIVE: DropKVNegativeScoreError}.get(code, DropKVError)
    raise cls(code, msg)


def _torch():
    import torch
    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise DropKVInvalidError(ERR_INVALID, f"unsupported dtype {t.dtype}")


def _shapes(q, k, v) -> Tuple[int, int, int, int, int]:
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise DropKVInvalidError(ERR_INVALID, "q must be [Hq, window, d], k and v [Hkv, n, d]")
    Hq, w, d = q.shape
    Hkv, n, dk = k.shape
    if tuple(v.shape) != (Hkv, n, dk) or dk != d:
        raise DropKVInvalidError(ERR_INVALID, "q/k/v shapes disagree")
    if not (q.dtype == k.dtype == v.dtype):
        raise DropKVInvalidError(ERR_INVALID, "q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise DropKVInvalidError(ERR_INVALID, "q, k, v must be contiguous GPU tensors")
    return Hq, Hkv, d, n, w


def score(q, k, v, *, pool_kernel: int, n_evict: int, stream=None):
    """DropKV scores and evict indices of one sequence.

    q [Hq, window, d], k/v [Hkv, n, d] (bf16 or fp32, contiguous, on the GPU).
    Returns (scores [Hkv, n] fp32 pooled with +inf on the window,
    evict_idx [Hkv, n_evict] int64 ascending).
    """
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    scores = torch.empty((Hkv, n), dtype=torch.float32, device=q.device)
    idx = torch.empty((Hkv, max(n_evict, 0)), dtype=torch.int64, device=q.device)
    fn = lib.dropkv_score if _dtype_code(q) == BF16 else lib.dropkv_score_f32
    rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq, Hkv, d, pool_kernel, n_evict,
            scores.data_ptr(), idx.data_ptr() if n_evict > 0 else None, _stream_handle(stream))
    _raise(rc)
    return scores, idx


def workspace_bytes(dtype_code: int, n: int, window: int, Hq: int, Hkv: int, d: int) -> int:
    return int(load_library().dropkv_workspace_bytes(dtype_code, n, window, Hq, Hkv, d))


def score_ex(q, k, v, *, pool_kernel: int, n_evict: int, workspace, status, scores=None,
             evict_idx=None, flags: int = 0, stream=None):
    """Asynchronous scoring into caller-owned workspace/status/outputs (no synchronisation).

    workspace: uint8 GPU tensor of >= workspace_bytes(...); status: int32 GPU
    tensor of one element that receives the STATUS_* bits. Returns (scores, evict_idx).
    """
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    if scores is None:
        scores = torch.empty((Hkv, n), dtype=torch.float32, device=q.device)
    if evict_idx is None:
        evict_idx = torch.empty((Hkv, max(n_evict, 0)), dtype=torch.int64, device=q.device)
    rc = lib.dropkv_score_ex(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq,
                             Hkv, d, pool_kernel, n_evict, scores.data_ptr(),
                             evict_idx.data_ptr() if n_evict > 0 else None, workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), status.data_ptr(),
                             flags, _stream_handle(stream))
    _raise(rc)
    return scores, evict_idx


def score_keep_ex(q, k, v, *, pool_kernel: int, n_evict: int, workspace, status, scores=None,
                  evict_idx=None, keep_idx=None, flags: int = 0, stream=None):
    """score_ex that also returns the kept token indices [Hkv, n - n_evict] (int64,
    ascending per head: the complement of evict_idx). Returns (scores, evict_idx, keep_idx)."""
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    if scores is None:
        scores = torch.empty((Hkv, n), dtype=torch.float32, device=q.device)
    if evict_idx is None:
        evict_idx = torch.empty((Hkv, max(n_evict, 0)), dtype=torch.int64, device=q.device)
    n_keep = n - n_evict
    if keep_idx is None:
        keep_idx = torch.empty((Hkv, max(n_keep, 0)), dtype=torch.int64, device=q.device)
    rc = lib.dropkv_score_keep_ex(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq,
                                  Hkv, d, pool_kernel, n_evict, scores.data_ptr(),
                                  evict_idx.data_ptr() if n_evict > 0 else None,
                                  keep_idx.data_ptr() if n_keep > 0 else None, workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), status.data_ptr(),
                                  flags, _stream_handle(stream))
    _raise(rc)
    return scores, evict_idx, keep_idx


NOALLOC_SCRATCH_BYTES = 64 << 20


def score_noalloc(q, k, v, *, pool_kernel: int, n_evict: int, status, scores, evict_idx, flags: int = 0,
                  stream=None):
    """dropkv_score_noalloc: scratch in the library's static device array, outputs
    and the device status word given by the caller (nothing is allocated here)."""
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    rc = lib.dropkv_score_noalloc(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq, Hkv, d,
                                  pool_kernel, n_evict, scores.data_ptr(),
                                  evict_idx.data_ptr() if n_evict > 0 else None, status.data_ptr(), flags,
                                  _stream_handle(stream))
    _raise(rc)
    return scores, evict_idx


def raw_scores(q, k, v, *, flags: int = 0, stream=None):
    """GQA-mean scores S [Hkv, n] before pooling and protection."""
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    S = torch.empty((Hkv, n), dtype=torch.float32, device=q.device)
    rc = lib.dropkv_raw_scores(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq,
                               Hkv, d, S.data_ptr(), flags, _stream_handle(stream))
    _raise(rc)
    return S


def row_stats(q, k, v, *, flags: int = 0, stream=None):
    """Per window row (h*window+i): (x_max, rest mass R, argmax or -1, output a [rows, d])."""
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    rows = Hq * w
    m = torch.empty(rows, dtype=torch.float32, device=q.device)
    rest = torch.empty(rows, dtype=torch.float32, device=q.device)
    arg = torch.empty(rows, dtype=torch.int32, device=q.device)
    a = torch.empty((rows, d), dtype=torch.float32, device=q.device)
    rc = lib.dropkv_row_stats(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq,
                              Hkv, d, m.data_ptr(), rest.data_ptr(), arg.data_ptr(), a.data_ptr(),
                              flags, _stream_handle(stream))
    _raise(rc)
    return m, rest, arg, a


def pass1_stats(q, k, v, *, stream=None):
    """bf16 inputs: the same per-row statistics as row_stats, through dropkv_pass1_stats."""
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    rows = Hq * w
    m = torch.empty(rows, dtype=torch.float32, device=q.device)
    rest = torch.empty(rows, dtype=torch.float32, device=q.device)
    arg = torch.empty(rows, dtype=torch.int32, device=q.device)
    a = torch.empty((rows, d), dtype=torch.float32, device=q.device)
    rc = lib.dropkv_pass1_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq, Hkv, d, m.data_ptr(),
                                rest.data_ptr(), arg.data_ptr(), a.data_ptr(), _stream_handle(stream))
    _raise(rc)
    return m, rest, arg, a


def select(S, *, window: int, pool_kernel: int, n_evict: int, stream=None):
    """Pool, protect and select on given raw scores S [Hkv, n] (fp32 GPU tensor, >= 0;
    a negative entry raises DropKVNegativeScoreError)."""
    torch = _torch()
    lib = load_library()
    Hkv, n = S.shape
    scores = torch.empty((Hkv, n), dtype=torch.float32, device=S.device)
    idx = torch.empty((Hkv, max(n_evict, 0)), dtype=torch.int64, device=S.device)
    rc = lib.dropkv_select(S.data_ptr(), n, window, Hkv, pool_kernel, n_evict, scores.data_ptr(),
                           idx.data_ptr() if n_evict > 0 else None, _stream_handle(stream))
    _raise(rc)
    return scores, idx


def score_from_stats(q, k, v, m, rest, argmax, a, *, pool_kernel: int, n_evict: int, stream=None,
                     workspace=None, status=None, scores=None, evict_idx=None):
    """Scores and evict indices from given window-row statistics (no pass 1):
    m, rest [Hq*window] fp32, argmax [Hq*window] int32, a [Hq*window, d] fp32,
    as row_stats returns them. bf16 q, k, v with d = 128. With `workspace`
    and `status` (device tensors, as for score_ex) the call is asynchronous."""
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    if _dtype_code(q) != BF16:
        raise DropKVInvalidError(ERR_INVALID, "score_from_stats takes bf16 q, k, v")
    rows = Hq * w
    for t, dt, shape in ((m, torch.float32, (rows,)), (rest, torch.float32, (rows,)),
                         (argmax, torch.int32, (rows,)), (a, torch.float32, (rows, d))):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
            raise DropKVInvalidError(ERR_INVALID, "row statistics must be contiguous GPU tensors "
                                     "m, rest [rows] fp32, argmax [rows] int32, a [rows, d] fp32")
    if scores is None:
        scores = torch.empty((Hkv, n), dtype=torch.float32, device=q.device)
    if evict_idx is None:
        evict_idx = torch.empty((Hkv, max(n_evict, 0)), dtype=torch.int64, device=q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq, Hkv, d, pool_kernel, n_evict,
            m.data_ptr(), rest.data_ptr(), argmax.data_ptr(), a.data_ptr(), scores.data_ptr(),
            evict_idx.data_ptr() if n_evict > 0 else None)
    if workspace is not None:
        rc = lib.dropkv_score_from_stats_ex(*ptrs, workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(),
                                            status.data_ptr(), _stream_handle(stream))
    else:
        rc = lib.dropkv_score_from_stats(*ptrs, _stream_handle(stream))
    _raise(rc)
    return scores, evict_idx


def prefill_attention(q_all, k, v, *, window: int, status=None, out_o=None, stream=None):
    """Causal prefill attention of bf16 q_all [Hq, n, d] against k, v [Hkv, n, d]:
    returns (o [Hq, n, d] bf16, m, rest, argmax, a) where the last four are the
    window rows' statistics in the layout score_from_stats takes. Asynchronous:
    `status` (int32 GPU tensor of one element, allocated if None) receives the
    STATUS_* bits."""
    torch = _torch()
    lib = load_library()
    if q_all.dim() != 3 or k.dim() != 3 or v.dim() != 3 or tuple(k.shape) != tuple(v.shape):
        raise DropKVInvalidError(ERR_INVALID, "q_all must be [Hq, n, d], k and v [Hkv, n, d]")
    Hq, n, d = q_all.shape
    Hkv = k.shape[0]
    if k.shape[1] != n or k.shape[2] != d:
        raise DropKVInvalidError(ERR_INVALID, "q_all/k/v shapes disagree")
    for t in (q_all, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise DropKVInvalidError(ERR_INVALID, "q_all, k, v must be contiguous bf16 GPU tensors")
    dev = q_all.device
    rows = Hq * window
    o = out_o if out_o is not None else torch.empty((Hq, n, d), dtype=torch.bfloat16, device=dev)
    m = torch.empty(rows, dtype=torch.float32, device=dev)
    rest = torch.empty(rows, dtype=torch.float32, device=dev)
    arg = torch.empty(rows, dtype=torch.int32, device=dev)
    a = torch.empty((rows, d), dtype=torch.float32, device=dev)
    st = status if status is not None else torch.zeros(1, dtype=torch.int32, device=dev)
    rc = lib.dropkv_prefill_attention(q_all.data_ptr(), k.data_ptr(), v.data_ptr(), n, window, Hq, Hkv, d,
                                      o.data_ptr(), m.data_ptr(), rest.data_ptr(), arg.data_ptr(), a.data_ptr(),
                                      st.data_ptr(), _stream_handle(stream))
    _raise(rc)
    return o, m, rest, arg, a


def compact(k, v, evict_idx, *, status=None, out_k=None, out_v=None, stream=None):
    """Cache compaction: the rows of k, v [Hkv, n, d] not listed in evict_idx
    [Hkv, n_evict] (int64, increasing per head) as out_k, out_v [Hkv, n - n_evict, d].

    With `status` (a device int32 tensor, cleared by the caller) the call is
    asynchronous and ORs STATUS_BAD_INDEX into it for an invalid list; without
    it the call synchronises and raises DropKVInvalidError for one.
    """
    torch = _torch()
    lib = load_library()
    if k.dim() != 3 or tuple(v.shape) != tuple(k.shape) or k.dtype != v.dtype:
        raise DropKVInvalidError(ERR_INVALID, "k and v must both be [Hkv, n, d] of one dtype")
    for t in (k, v, evict_idx):
        if not t.is_cuda or not t.is_contiguous():
            raise DropKVInvalidError(ERR_INVALID, "k, v and evict_idx must be contiguous GPU tensors")
    Hkv, n, d = k.shape
    if evict_idx.dtype != torch.int64 or evict_idx.dim() != 2 or evict_idx.shape[0] != Hkv:
        raise DropKVInvalidError(ERR_INVALID, "evict_idx must be int64 [Hkv, n_evict]")
    n_evict = evict_idx.shape[1]
    n_keep = n - n_evict
    if out_k is None:
        out_k = torch.empty((Hkv, max(n_keep, 0), d), dtype=k.dtype, device=k.device)
    if out_v is None:
        out_v = torch.empty((Hkv, max(n_keep, 0), d), dtype=k.dtype, device=k.device)
    sync = status is None
    if sync:
        status = torch.zeros(1, dtype=torch.int32, device=k.device)
    rc = lib.dropkv_compact(_dtype_code(k), k.data_ptr(), v.data_ptr(), n, Hkv, d,
                            evict_idx.data_ptr() if n_evict > 0 else None, n_evict,
                            out_k.data_ptr() if n_keep > 0 else None,
                            out_v.data_ptr() if n_keep > 0 else None, status.data_ptr(),
                            _stream_handle(stream))
    _raise(rc)
    if sync and int(status.item()) & STATUS_BAD_INDEX:
        raise DropKVInvalidError(ERR_INVALID, "evict_idx is not strictly increasing inside [0, n)")
    return out_k, out_v


def compact_kept(k, v, keep_idx, *, status=None, out_k=None, out_v=None, stream=None):
    """Cache compaction from a kept list: out_k, out_v [Hkv, n_keep, d] = the rows
    keep_idx [Hkv, n_keep] (int64, strictly increasing per head) of k, v [Hkv, n, d].

    With `status` (a device int32 tensor, cleared by the caller) the call is
    asynchronous and ORs STATUS_BAD_INDEX into it for an invalid list; without
    it the call synchronises and raises DropKVInvalidError for one.
    """
    torch = _torch()
    lib = load_library()
    if k.dim() != 3 or tuple(v.shape) != tuple(k.shape) or k.dtype != v.dtype:
        raise DropKVInvalidError(ERR_INVALID, "k and v must both be [Hkv, n, d] of one dtype")
    for t in (k, v, keep_idx):
        if not t.is_cuda or not t.is_contiguous():
            raise DropKVInvalidError(ERR_INVALID, "k, v and keep_idx must be contiguous GPU tensors")
    Hkv, n, d = k.shape
    if keep_idx.dtype != torch.int64 or keep_idx.dim() != 2 or keep_idx.shape[0] != Hkv:
        raise DropKVInvalidError(ERR_INVALID, "keep_idx must be int64 [Hkv, n_keep]")
    n_keep = keep_idx.shape[1]
    if out_k is None:
        out_k = torch.empty((Hkv, n_keep, d), dtype=k.dtype, device=k.device)
    if out_v is None:
        out_v = torch.empty((Hkv, n_keep, d), dtype=k.dtype, device=k.device)
    sync = status is None
    if sync:
        status = torch.zeros(1, dtype=torch.int32, device=k.device)
    rc = lib.dropkv_compact_kept(_dtype_code(k), k.data_ptr(), v.data_ptr(), n, Hkv, d,
                                 keep_idx.data_ptr() if n_keep > 0 else None, n_keep,
                                 out_k.data_ptr() if n_keep > 0 else None,
                                 out_v.data_ptr() if n_keep > 0 else None, status.data_ptr(),
                                 _stream_handle(stream))
    _raise(rc)
    if sync and int(status.item()) & STATUS_BAD_INDEX:
        raise DropKVInvalidError(ERR_INVALID, "keep_idx is not strictly increasing inside [0, n)")
    return out_k, out_v


class DecodeScorer:
    """Decode-time rescoring of one sequence's cache (dropkv_decode_* calls).

    The cache is the caller's k, v [Hkv, n_max, d] bf16 tensors, of which the
    first n token rows of each head are valid; the scorer owns the device
    state (sized for n_max) and a device status word. Calls are asynchronous
    on the current stream; check() synchronises and raises on a recorded
    singular / non-finite row. After step(..., deferred=True) the newest
    position's terms are pending; the reading calls (raw_scores,
    raw_scores_f64, select) flush them first with the k, v of that step.
    """

    def __init__(self, *, n_max: int, window: int, Hq: int, Hkv: int, d: int, device=None):
        torch = _torch()
        self.lib = load_library()
        self.n_max, self.window, self.Hq, self.Hkv, self.d = n_max, window, Hq, Hkv, d
        nbytes = self.lib.dropkv_decode_state_bytes(n_max, window, Hq, Hkv, d)
        if nbytes == 0:
            raise DropKVInvalidError(ERR_INVALID, "unsupported decode shape (bf16, d = 128)")
        self.state = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device=self.state.device)
        self.n = 0
        self._pending_kv = None  # (k, v) of a deferred step whose terms are not in S yet

    def _kv(self, k, v):
        torch = _torch()
        want = (self.Hkv, self.n_max, self.d)
        for t in (k, v):
            if tuple(t.shape) != want or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise DropKVInvalidError(ERR_INVALID, f"k and v must be contiguous bf16 GPU tensors {list(want)}")

    def _args(self):
        return (self.n_max, self.window, self.Hq, self.Hkv, self.d)

    def init(self, q, k, v, n: int, stream=None):
        """Score the first n tokens; q [Hq, window, d] are the last window positions' query rows."""
        self._kv(k, v)
        if tuple(q.shape) != (self.Hq, self.window, self.d) or q.dtype != k.dtype or not q.is_contiguous():
            raise DropKVInvalidError(ERR_INVALID, "q must be contiguous bf16 [Hq, window, d]")
        _raise(self.lib.dropkv_decode_init(q.data_ptr(), k.data_ptr(), v.data_ptr(), n, *self._args(),
                                           self.state.data_ptr(), self.state.numel(), self.status.data_ptr(),
                                           _stream_handle(stream)))
        self.n = n
        self._pending_kv = None

    def step(self, q_new, k, v, stream=None, *, deferred: bool = False):
        """Append one token: its key and value are already at row self.n of k and v; q_new [Hq, d].

        deferred=True takes the single-pass step (one read of the cache): the
        new position's terms stay pending until the next step, a flush or a
        reading call.
        """
        self._kv(k, v)
        if tuple(q_new.shape) != (self.Hq, self.d) or q_new.dtype != k.dtype or not q_new.is_contiguous():
            raise DropKVInvalidError(ERR_INVALID, "q_new must be contiguous bf16 [Hq, d]")
        n = self.n + 1
        fn = self.lib.dropkv_decode_step_deferred if deferred else self.lib.dropkv_decode_step
        _raise(fn(q_new.data_ptr(), k.data_ptr(), v.data_ptr(), n, *self._args(), self.state.data_ptr(),
                  self.state.numel(), self.status.data_ptr(), _stream_handle(stream)))
        self.n = n
        self._pending_kv = (k, v) if deferred else None

    def flush(self, stream=None):
        """Add the terms a deferred step left pending (no-op if none)."""
        if self._pending_kv is None:
            return
        k, v = self._pending_kv
        _raise(self.lib.dropkv_decode_flush(k.data_ptr(), v.data_ptr(), self.n, *self._args(),
                                            self.state.data_ptr(), self.state.numel(), _stream_handle(stream)))
        self._pending_kv = None

    def rebuild(self, k, v, stream=None):
        """Recompute the kept score from the stored window rows (nothing stays pending)."""
        self._kv(k, v)
        _raise(self.lib.dropkv_decode_rebuild(k.data_ptr(), v.data_ptr(), self.n, *self._args(),
                                              self.state.data_ptr(), self.state.numel(), self.status.data_ptr(),
                                              _stream_handle(stream)))
        self._pending_kv = None

    def raw_scores(self, stream=None):
        """The kept raw score as fp32 [Hkv, n]."""
        torch = _torch()
        self.flush(stream)
        out = torch.empty((self.Hkv, self.n), dtype=torch.float32, device=self.state.device)
        _raise(self.lib.dropkv_decode_scores(self.state.data_ptr(), self.state.numel(), self.n, *self._args(),
                                             out.data_ptr(), _stream_handle(stream)))
        return out

    def raw_scores_f64(self):
        """The kept fp64 score [Hkv, n] (a view into the state: S64 comes first in its layout)."""
        torch = _torch()
        self.flush()
        S64 = self.state[: 8 * self.Hkv * self.n_max].view(torch.float64).view(self.Hkv, self.n_max)
        return S64[:, : self.n]

    def select(self, *, pool_kernel: int, n_evict: int, stream=None):
        """Re-eviction on the kept score: (pooled scores [Hkv, n], evict_idx [Hkv, n_evict])."""
        torch = _torch()
        self.flush(stream)
        scores = torch.empty((self.Hkv, self.n), dtype=torch.float32, device=self.state.device)
        idx = torch.empty((self.Hkv, max(n_evict, 0)), dtype=torch.int64, device=self.state.device)
        _raise(self.lib.dropkv_decode_select(self.state.data_ptr(), self.state.numel(), self.n, *self._args(),
                                             pool_kernel, n_evict, scores.data_ptr(),
                                             idx.data_ptr() if n_evict > 0 else None, self.status.data_ptr(),
                                             _stream_handle(stream)))
        return scores, idx

    def check(self):
        """Synchronise and raise if a call recorded a singular or non-finite row."""
        word = int(self.status.item())
        if word & STATUS_SINGULAR:
            raise DropKVSingularError(ERR_SINGULAR, "a window row has a probability that rounds to 1 (singular)")
        if word & STATUS_NONFINITE:
            raise DropKVNonFiniteError(ERR_NONFINITE, "non-finite inputs or scores")


def stage_times(q, k, v, *, pool_kernel: int, n_evict: int, flags: int = 0, stream=None):
    """One scoring call with each stage's begin and end time recorded.

    Returns (scores, evict_idx, [(stage name, milliseconds), ...]).
    """
    torch = _torch()
    lib = load_library()
    Hq, Hkv, d, n, w = _shapes(q, k, v)
    scores = torch.empty((Hkv, n), dtype=torch.float32, device=q.device)
    idx = torch.empty((Hkv, max(n_evict, 0)), dtype=torch.int64, device=q.device)
    ms = (ctypes.c_float * 16)()
    names = ctypes.create_string_buffer(512)
    count = ctypes.c_int32(0)
    rc = lib.dropkv_stage_times(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), n, w, Hq,
                                Hkv, d, pool_kernel, n_evict, scores.data_ptr(),
                                idx.data_ptr() if n_evict > 0 else None, flags,
                                ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(names, ctypes.c_void_p),
                                512, ctypes.cast(ctypes.pointer(count), ctypes.c_void_p),
                                _stream_handle(stream))
    _raise(rc)
    labels = names.value.decode().split(",") if count.value else []
    return scores, idx, [(labels[i], float(ms[i])) for i in range(count.value)]


def stage_log():
    """Mean per-stage milliseconds of the calls logged with FLAG_STAGE_LOG since the last read.

    Returns (calls, [(stage name, milliseconds), ...]) and empties the log.
    """
    lib = load_library()
    ms = (ctypes.c_float * 16)()
    names = ctypes.create_string_buffer(512)
    count = ctypes.c_int32(0)
    calls = ctypes.c_int32(0)
    rc = lib.dropkv_stage_log(ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(names, ctypes.c_void_p), 512,
                              ctypes.cast(ctypes.pointer(count), ctypes.c_void_p),
                              ctypes.cast(ctypes.pointer(calls), ctypes.c_void_p))
    _raise(rc)
    labels = names.value.decode().split(",") if count.value else []
    return calls.value, [(labels[i], float(ms[i])) for i in range(count.value)]


def uses_mfma(dtype_code: int, d: int) -> bool:
    return bool(load_library().dropkv_uses_mfma(dtype_code, d))


def version() -> str:
    return load_library().dropkv_version().decode()
