"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/cobs.h, and rejects invalid calls on the host before any
HIP call (so nothing is enqueued)."""
import ctypes
import os
import re

import pytest

from block_sparse_long_compressed_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "cobs.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cobs_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "cobs_sparse_attn_decode" in names and len(names) >= 8
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in B._SIGNATURES, f"binding lacks {n}"


def good():
    return B.make_params(128, 64, 4, 16, window=512, cmp_len=32, cmp_stride=16)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, B.COBS_ERR_UNSUPPORTED),
    ("n_kv_heads", 3, B.COBS_ERR_INVALID_ARG),
    ("n_kv_heads", 2, B.COBS_ERR_UNSUPPORTED),       # group 32
    ("n_q_heads", 0, B.COBS_ERR_INVALID_ARG),
    ("top_k", 0, B.COBS_ERR_INVALID_ARG),
    ("top_k", 65, B.COBS_ERR_INVALID_ARG),
    ("window", -1, B.COBS_ERR_INVALID_ARG),
    ("block_size", 128, B.COBS_ERR_UNSUPPORTED),
    ("cmp_len", 64, B.COBS_ERR_UNSUPPORTED),
    ("so_kind", 5, B.COBS_ERR_INVALID_ARG),
    ("alpha", -0.5, B.COBS_ERR_INVALID_ARG),
    ("alpha", float("nan"), B.COBS_ERR_INVALID_ARG),
    ("scale", float("inf"), B.COBS_ERR_INVALID_ARG),
    ("kv_dtype", 7, B.COBS_ERR_INVALID_ARG),
])
def test_invalid_params_rejected(field, value, status):
    p = good()
    setattr(p, field, value)
    assert B.cobs_validate_params(p) == status
    assert B.cobs_workspace_bytes(p, 1, 1024) == 0


@pytest.mark.parametrize("kind", [B.COBS_SO_LOWRANK, B.COBS_SO_LOWRANK_FP4])
def test_lowrank_rank_bounds(kind):
    p = good()
    p.so_kind = kind
    for r, st in ((0, B.COBS_ERR_INVALID_ARG), (1, B.COBS_OK), (8, B.COBS_OK), (9, B.COBS_ERR_INVALID_ARG)):
        p.rank = r
        assert B.cobs_validate_params(p) == st


def test_summary_shapes():
    p = good()
    sh = B.cobs_summary_shapes(p, 2, 1000)
    assert sh["nb_max"] == 16 and sh["nc_max"] == (1000 - 32) // 16 + 1
    assert sh["mu_bytes"] == 2 * 4 * 16 * 128 * 4 == sh["so_bytes"]
    assert sh["pooled_bytes"] == 2 * 4 * sh["nc_max"] * 128 * 2
    p.cmp_len = 0
    assert B.cobs_summary_shapes(p, 1, 1000)["nc_max"] == 0
    p.cmp_len = 32
    assert B.cobs_summary_shapes(p, 1, 20)["nc_max"] == 0
    p.so_kind, p.rank = B.COBS_SO_LOWRANK, 4
    assert B.cobs_summary_shapes(p, 1, 128)["so_bytes"] == 4 * 2 * 4 * 128 * 4


@pytest.mark.parametrize("d,rank,record", [(128, 4, 272), (128, 1, 80), (128, 8, 544), (64, 3, 112), (64, 1, 48)])
def test_summary_shapes_fp4(d, rank, record):
    # per vector d/2 code bytes and d/32 exponent bytes; the record is padded to 16
    p = B.make_params(d, 8, 2, 8, so_kind=B.COBS_SO_LOWRANK_FP4, rank=rank)
    sh = B.cobs_summary_shapes(p, 3, 1000)
    assert sh["mu_bytes"] == 3 * 2 * 16 * d * 2                 # bf16 means
    assert sh["so_bytes"] == 3 * 2 * 16 * record


def test_workspace_grows_with_problem_and_rejects_bad_sizes():
    p = good()
    a = B.cobs_workspace_bytes(p, 1, 32768)
    b = B.cobs_workspace_bytes(p, 32, 32768)
    assert 0 < a < b and a % 256 == 0
    assert B.cobs_workspace_bytes(p, 0, 1024) == 0
    assert B.cobs_workspace_bytes(p, 1, 0) == 0
    assert B.cobs_workspace_bytes(p, 1, 64 * 4096 + 1) == 0


def test_null_pointers_and_small_workspace_rejected_before_any_hip_call():
    lib = B.lib()
    p = good()
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    st = lib.cobs_sparse_attn_decode(ctypes.byref(p), 1, 1024, None, fake, fake, fake, fake, fake, fake, fake,
                                     None, None, None, fake, fake, 1 << 30, None)
    assert st == B.COBS_ERR_INVALID_ARG
    st = lib.cobs_sparse_attn_decode(ctypes.byref(p), 1, 1024, fake, fake, fake, fake, fake, fake, fake, fake,
                                     None, None, None, fake, fake, 16, None)
    assert st == B.COBS_ERR_WORKSPACE
    st = lib.cobs_build_summaries(ctypes.byref(p), 1, 1024, fake, fake, fake, fake, fake, None, None, None)
    assert st == B.COBS_ERR_INVALID_ARG                   # pooled outputs missing
    st = lib.cobs_select_topk(ctypes.byref(p), 1, 1024, fake, 2, -1, fake, fake, fake, fake, None, fake,
                              1 << 30, None)
    assert st == B.COBS_ERR_INVALID_ARG                   # decode takes one token
    st = lib.cobs_sparse_attn_prefill(ctypes.byref(p), 1024, 10, 1020, fake, fake, fake, fake, fake, fake, fake,
                                      None, None, fake, fake, 1 << 30, None)
    assert st == B.COBS_ERR_INVALID_ARG                   # tokens run past the prefix
    st = lib.cobs_update_summaries(ctypes.byref(p), 1, 1024, fake, fake, 0, fake, fake, fake, fake, fake, fake,
                                   None)
    assert st == B.COBS_ERR_INVALID_ARG                   # max_append must be >= 1
    st = lib.cobs_update_summaries(ctypes.byref(p), 1, 1024, None, fake, 1, fake, fake, fake, fake, fake, fake,
                                   None)
    assert st == B.COBS_ERR_INVALID_ARG                   # old lengths missing
    st = lib.cobs_update_summaries(ctypes.byref(p), 1, 1024, fake, fake, 1, fake, fake, fake, fake, None, None,
                                   None)
    assert st == B.COBS_ERR_INVALID_ARG                   # pooled outputs missing


def test_status_strings():
    assert B.status_string(0) == "ok"
    assert "workspace" in B.status_string(3)
    assert B.status_string(99) == "unknown status"


def test_subspace_params_validated():
    p = B.make_params(128, 8, 2, 8, so_kind=B.COBS_SO_LOWRANK, rank=4)
    fake = 0x1000                                  # never dereferenced by validation
    p.subspace_dim, p.subspace = 85, fake
    assert B.cobs_validate_params(p) == B.COBS_OK
    p.subspace = None
    assert B.cobs_validate_params(p) == B.COBS_ERR_INVALID_ARG     # dimension without a subspace
    p.subspace, p.subspace_dim = fake, 129
    assert B.cobs_validate_params(p) == B.COBS_ERR_INVALID_ARG     # more than head_dim
    p.subspace_dim = -1
    assert B.cobs_validate_params(p) == B.COBS_ERR_INVALID_ARG
    p.subspace_dim, p.so_kind, p.rank = 40, B.COBS_SO_DIAG, 0
    assert B.cobs_validate_params(p) == B.COBS_ERR_INVALID_ARG     # diagonal kind has no vectors
    p.subspace_dim = 0
    assert B.cobs_validate_params(p) == B.COBS_OK                  # pointer ignored when off


@pytest.mark.parametrize("kind,s,so_bytes", [
    (B.COBS_SO_LOWRANK, 85, 3 * 2 * 16 * 4 * 96 * 4),     # vectors of length 96 (85 rounded up to 32)
    (B.COBS_SO_LOWRANK, 32, 3 * 2 * 16 * 4 * 32 * 4),
    (B.COBS_SO_LOWRANK_FP4, 85, 3 * 2 * 16 * 208),         # 4 * (48 + 3) = 204 -> 208
    (B.COBS_SO_LOWRANK_FP4, 20, 3 * 2 * 16 * 80),          # 4 * (16 + 1) = 68 -> 80
])
def test_summary_shapes_subspace(kind, s, so_bytes):
    p = B.make_params(128, 8, 2, 8, so_kind=kind, rank=4)
    p.subspace_dim, p.subspace = s, 0x1000
    sh = B.cobs_summary_shapes(p, 3, 1000)
    assert sh["so_bytes"] == so_bytes
    assert sh["mu_bytes"] == 3 * 2 * 16 * 128 * (2 if kind == B.COBS_SO_LOWRANK_FP4 else 4)


def test_query_subspace_rejects_bad_calls():
    lib = B.lib()
    p = B.make_params(128, 8, 2, 8, so_kind=B.COBS_SO_LOWRANK, rank=4)
    p.subspace_dim = 16
    n = lib.cobs_query_subspace_workspace_bytes(ctypes.byref(p))
    assert n == 2 * 2 * 128 * 128 * 8
    fake = ctypes.c_void_p(0x1000)
    assert lib.cobs_query_subspace(ctypes.byref(p), 0, fake, fake, fake, n, None) == B.COBS_ERR_INVALID_ARG
    assert lib.cobs_query_subspace(ctypes.byref(p), 10, fake, None, fake, n, None) == B.COBS_ERR_INVALID_ARG
    assert lib.cobs_query_subspace(ctypes.byref(p), 10, fake, fake, fake, n - 1, None) == B.COBS_ERR_WORKSPACE
    p.subspace_dim = 0
    assert lib.cobs_query_subspace(ctypes.byref(p), 10, fake, fake, fake, n, None) == B.COBS_ERR_INVALID_ARG
    p.subspace_dim, p.so_kind, p.rank = 16, B.COBS_SO_DIAG, 0
    assert lib.cobs_query_subspace(ctypes.byref(p), 10, fake, fake, fake, n, None) == B.COBS_ERR_INVALID_ARG


def test_static_decode_rejects_oversized_workspace_on_the_host():
    # a configuration whose workspace exceeds the library's static array: rejected
    # before any HIP call (the tensors are never looked at)
    p = B.make_params(128, 32, 8, 32, window=1024, cmp_len=32, cmp_stride=16, so_kind=B.COBS_SO_LOWRANK, rank=4)
    assert B.cobs_workspace_bytes(p, 256, 131072) > B.COBS_STATIC_SCRATCH_BYTES
    st = B.lib().cobs_sparse_attn_decode_static(ctypes.byref(p), 256, 131072, None, None, None, None, None, None,
                                                None, None, None, None, None, None, None)
    assert st == B.COBS_ERR_WORKSPACE
    bad = good()
    bad.head_dim = 96
    st = B.lib().cobs_sparse_attn_decode_static(ctypes.byref(bad), 1, 1024, None, None, None, None, None, None,
                                                None, None, None, None, None, None, None)
    assert st == B.COBS_ERR_UNSUPPORTED


def test_decode_status_argument_checks_on_the_host():
    p = good()
    flags = ctypes.c_uint32()
    assert B.lib().cobs_decode_status(ctypes.byref(p), 1, 1024, None, 0, None, None) == B.COBS_ERR_INVALID_ARG
    assert B.lib().cobs_decode_status(ctypes.byref(p), 1, 1024, None, 64, ctypes.byref(flags),
                                      None) == B.COBS_ERR_INVALID_ARG
    ws_bytes = B.cobs_workspace_bytes(p, 1, 1024)
    buf = ctypes.create_string_buffer(16)
    assert B.lib().cobs_decode_status(ctypes.byref(p), 1, 1024, buf, ws_bytes - 1, ctypes.byref(flags),
                                      None) == B.COBS_ERR_WORKSPACE
