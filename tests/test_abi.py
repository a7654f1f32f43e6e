"""The C-ABI library loads and exports every symbol include/dropkv.h declares.

No compute call is made here: only pure host-side entry points (workspace
sizing, argument validation that rejects before any HIP call).
"""

import ctypes
import os
import re

import pytest

import kv_cache_eviction_pass1_amd as K
from kv_cache_eviction_pass1_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dropkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dropkv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libdropkv.so is not built (run __graft_entry__.build())")
    return K.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES, f"binding lacks a signature for {name}"


def test_binding_covers_only_declared_symbols():
    assert set(binding.SIGNATURES) == set(declared_functions())


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    for name, val in [("DROPKV_OK", 0), ("DROPKV_ERR_INVALID", -1), ("DROPKV_ERR_SINGULAR", -2),
                      ("DROPKV_ERR_NONFINITE", -3), ("DROPKV_ERR_DEVICE", -4),
                      ("DROPKV_ERR_NEGATIVE", -5), ("DROPKV_STATUS_NEGATIVE", 16)]:
        assert re.search(rf"{name}\s*=\s*{val}\b", text), name
    assert (binding.OK, binding.ERR_INVALID, binding.ERR_SINGULAR, binding.ERR_NONFINITE,
            binding.ERR_DEVICE, binding.ERR_NEGATIVE, binding.STATUS_NEGATIVE) == (0, -1, -2, -3, -4, -5, 16)
    assert re.search(r"DROPKV_BF16\s*=\s*0", text) and re.search(r"DROPKV_F32\s*=\s*1", text)


def test_workspace_sizing_is_host_only(lib):
    llama = lib.dropkv_workspace_bytes(0, 131072, 64, 32, 8, 128)
    assert llama > 4 * 8 * 131072  # at least the raw scores
    assert llama < 512 << 20       # no materialised attention (w*n per head)
    assert lib.dropkv_workspace_bytes(0, 10, 10, 4, 2, 8) == 0   # window >= n
    assert lib.dropkv_workspace_bytes(0, 22, 3, 4, 3, 8) == 0    # Hq % Hkv
    assert lib.dropkv_workspace_bytes(0, 22, 3, 4, 2, 300) == 0  # d > 256
    assert lib.dropkv_workspace_bytes(7, 22, 3, 4, 2, 8) == 0    # dtype


@pytest.mark.parametrize("bad", [
    dict(window=0), dict(window=22), dict(Hkv=3), dict(d=0), dict(d=257),
    dict(pool_kernel=4), dict(pool_kernel=0), dict(n_evict=-1), dict(n_evict=20),
])
def test_invalid_arguments_rejected_before_any_device_call(lib, bad):
    args = dict(n=22, window=3, Hq=4, Hkv=2, d=8, pool_kernel=3, n_evict=7)
    args.update(bad)
    rc = lib.dropkv_score(None, None, None, args["n"], args["window"], args["Hq"], args["Hkv"],
                          args["d"], args["pool_kernel"], args["n_evict"], None, None, None)
    assert rc == binding.ERR_INVALID
    assert lib.dropkv_last_error().decode()


def test_boundary_aliases_share_the_error_text(lib):
    rc = lib.dropkv_score(None, None, None, 22, 3, 4, 2, 8, 3, 7, None, None, None)
    assert rc == binding.ERR_INVALID
    assert lib.dropkv_last_error_string() == lib.dropkv_last_error() != b""
    rc = lib.dropkv_pass1_stats(None, None, None, 22, 0, 4, 2, 128, None, None, None, None, None)
    assert rc == binding.ERR_INVALID


def test_null_pointers_rejected(lib):
    rc = lib.dropkv_score(None, None, None, 22, 3, 4, 2, 8, 3, 7, None, None, None)
    assert rc == binding.ERR_INVALID
    assert b"null" in lib.dropkv_last_error()


def test_package_import_does_not_require_gpu():
    # importing and loading the library work without a GPU; compute calls would raise
    assert callable(K.score) and callable(K.score_ex)
    assert ctypes.sizeof(ctypes.c_void_p) == 8


def test_kept_list_entry_points_reject_bad_arguments_on_the_host(lib):
    # scoring with the kept list: a missing kept-list output while tokens are kept
    rc = lib.dropkv_score_keep_ex(0, None, None, None, 22, 3, 4, 2, 8, 3, 7, None, None, None, None, 0, None, 0,
                                  None)
    assert rc == binding.ERR_INVALID
    assert b"out_keep_idx" in lib.dropkv_last_error()
    # compaction from a kept list: bad dtype, more kept tokens than tokens, bad sizes
    assert lib.dropkv_compact_kept(7, None, None, 100, 2, 8, None, 10, None, None, None, None) == binding.ERR_INVALID
    assert lib.dropkv_compact_kept(0, None, None, 100, 2, 8, None, 101, None, None, None, None) == binding.ERR_INVALID
    assert b"n_keep" in lib.dropkv_last_error()
    assert lib.dropkv_compact_kept(0, None, None, 100, 0, 8, None, 10, None, None, None, None) == binding.ERR_INVALID
    assert lib.dropkv_compact_kept(0, None, None, 0, 2, 8, None, 0, None, None, None, None) == binding.ERR_INVALID
