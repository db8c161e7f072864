"""Python binding of libcobs.so: argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the method; torch tensors provide device memory and the current
HIP stream.  If the library has not been built the first call raises, so no
code path can fall back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcobs.so")

COBS_OK, COBS_ERR_INVALID_ARG, COBS_ERR_UNSUPPORTED, COBS_ERR_WORKSPACE, COBS_ERR_HIP = range(5)
COBS_BF16, COBS_F32 = 0, 1
COBS_SO_DIAG, COBS_SO_LOWRANK, COBS_SO_LOWRANK_FP4 = 0, 1, 2


class cobs_params(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("cmp_len", ctypes.c_int32),
        ("cmp_stride", ctypes.c_int32),
        ("so_kind", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("kv_dtype", ctypes.c_int32),
        ("subspace_dim", ctypes.c_int32),
        ("subspace", ctypes.c_void_p),
    ]


class CobsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


_lib = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_P = ctypes.POINTER(cobs_params)

_SIGNATURES = {
    "cobs_status_string": (ctypes.c_char_p, [_i32]),
    "cobs_validate_params": (_i32, [_P]),
    "cobs_summary_shapes": (_i32, [_P, _i32, _i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                   ctypes.POINTER(_sz), ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "cobs_workspace_bytes": (_sz, [_P, _i32, _i32, _i32]),
    "cobs_build_summaries": (_i32, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "cobs_select_topk": (_i32, [_P, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "cobs_update_summaries": (_i32, [_P, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "cobs_select_topk_exact": (_i32, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "cobs_sparse_attn_decode": (_i32, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _sz, _vp]),
    "cobs_sparse_attn_prefill": (_i32, [_P, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _sz, _vp]),
    "cobs_decode_status": (_i32, [_P, _i32, _i32, _vp, _sz, ctypes.POINTER(ctypes.c_uint32), _vp]),
    "cobs_set_poll_limit": (None, [ctypes.c_uint32]),
    "cobs_sparse_attn_decode_static": (_i32, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _vp]),
    "cobs_query_subspace_workspace_bytes": (_sz, [_P]),
    "cobs_query_subspace": (_i32, [_P, _i32, _vp, _vp, _vp, _sz, _vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_long_compressed_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().cobs_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != COBS_OK:
        raise CobsError(fn, status)


def make_params(head_dim: int, n_q_heads: int, n_kv_heads: int, top_k: int, window: int = 0,
                cmp_len: int = 0, cmp_stride: int = 16, so_kind: int = COBS_SO_DIAG, rank: int = 0,
                alpha: float = 1.0, scale: float = 0.0, kv_dtype: int = COBS_BF16,
                block_size: int = 64, subspace: Optional[torch.Tensor] = None) -> cobs_params:
    """Method parameters.  `subspace` ([H_kv][s][d] fp32 on the device) turns on the
    query-subspace projection with s = its second dimension; the caller keeps the
    tensor alive while the parameters are in use."""
    p = cobs_params(head_dim, n_q_heads, n_kv_heads, block_size, top_k, window, cmp_len, cmp_stride,
                    so_kind, rank, alpha, scale, kv_dtype, 0, None)
    if subspace is not None:
        set_subspace(p, subspace)
    return p


def set_subspace(p: cobs_params, P: Optional[torch.Tensor]) -> None:
    """Point the parameters at a query subspace [H_kv][s][d] (fp32, contiguous), or
    turn the projection off with None."""
    if P is None:
        p.subspace_dim, p.subspace = 0, None
        return
    if P.dtype != torch.float32 or P.dim() != 3 or not P.is_contiguous():
        raise ValueError("subspace must be a contiguous fp32 [H_kv][s][d] tensor")
    p.subspace_dim, p.subspace = P.shape[1], P.data_ptr()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libcobs must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def cobs_validate_params(p: cobs_params) -> int:
    return lib().cobs_validate_params(ctypes.byref(p))


def cobs_summary_shapes(p: cobs_params, batch: int, max_len: int) -> dict:
    nb, nc = ctypes.c_int64(), ctypes.c_int64()
    mb, sb, pb = _sz(), _sz(), _sz()
    _check("cobs_summary_shapes", lib().cobs_summary_shapes(ctypes.byref(p), batch, max_len, ctypes.byref(nb),
                                                            ctypes.byref(nc), ctypes.byref(mb), ctypes.byref(sb),
                                                            ctypes.byref(pb)))
    return {"nb_max": nb.value, "nc_max": nc.value, "mu_bytes": mb.value, "so_bytes": sb.value,
            "pooled_bytes": pb.value}


def cobs_workspace_bytes(p: cobs_params, batch: int, max_len: int, n_q_tokens: int = 1) -> int:
    return lib().cobs_workspace_bytes(ctypes.byref(p), batch, max_len, n_q_tokens)


def cobs_build_summaries(p: cobs_params, seq_lens, K, V, mu, so, kc=None, vc=None, stream=None) -> None:
    batch, max_len = K.shape[0], K.shape[2]
    _check("cobs_build_summaries", lib().cobs_build_summaries(
        ctypes.byref(p), batch, max_len, _ptr(seq_lens), _ptr(K), _ptr(V), _ptr(mu), _ptr(so), _ptr(kc),
        _ptr(vc), _stream(stream)))


def cobs_update_summaries(p: cobs_params, old_lens, new_lens, max_append: int, K, V, mu, so, kc=None, vc=None,
                          stream=None) -> None:
    batch, max_len = K.shape[0], K.shape[2]
    _check("cobs_update_summaries", lib().cobs_update_summaries(
        ctypes.byref(p), batch, max_len, _ptr(old_lens), _ptr(new_lens), max_append, _ptr(K), _ptr(V), _ptr(mu),
        _ptr(so), _ptr(kc), _ptr(vc), _stream(stream)))


def cobs_select_topk_exact(p: cobs_params, seq_lens, Q, K, sel, ws, sel_score=None, stream=None) -> None:
    batch, max_len = K.shape[0], K.shape[2]
    _check("cobs_select_topk_exact", lib().cobs_select_topk_exact(
        ctypes.byref(p), batch, max_len, _ptr(seq_lens), _ptr(Q), _ptr(K), _ptr(sel), _ptr(sel_score), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def cobs_select_topk(p: cobs_params, seq_lens, Q, mu, so, sel, ws, sel_score=None, max_len: int = 0,
                     q_pos0: int = -1, stream=None) -> None:
    batch, tokens = Q.shape[0], Q.shape[1]
    _check("cobs_select_topk", lib().cobs_select_topk(
        ctypes.byref(p), batch, max_len, _ptr(seq_lens), tokens, q_pos0, _ptr(Q), _ptr(mu), _ptr(so), _ptr(sel),
        _ptr(sel_score), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def cobs_sparse_attn_decode(p: cobs_params, seq_lens, Q, K, V, mu, so, kc, vc, gates, out, ws,
                            sel_in=None, sel_out=None, stream=None) -> None:
    batch, max_len = K.shape[0], K.shape[2]
    _check("cobs_sparse_attn_decode", lib().cobs_sparse_attn_decode(
        ctypes.byref(p), batch, max_len, _ptr(seq_lens), _ptr(Q), _ptr(K), _ptr(V), _ptr(mu), _ptr(so),
        _ptr(kc), _ptr(vc), _ptr(gates), _ptr(sel_in), _ptr(sel_out), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


COBS_STATUS_WAIT_GAVE_UP = 1


def cobs_decode_status(p: cobs_params, batch: int, max_len: int, ws, stream=None) -> int:
    """Status bits of the decode steps run on ws since the last query (synchronises);
    ws=None reads the array of cobs_sparse_attn_decode_static."""
    flags = ctypes.c_uint32()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("cobs_decode_status", lib().cobs_decode_status(ctypes.byref(p), batch, max_len, _ptr(ws), nbytes,
                                                          ctypes.byref(flags), _stream(stream)))
    return flags.value


COBS_STATIC_SCRATCH_BYTES = 16 << 20


def cobs_sparse_attn_decode_static(p: cobs_params, seq_lens, Q, K, V, mu, so, kc, vc, gates, out,
                                   sel_in=None, sel_out=None, stream=None) -> None:
    """cobs_sparse_attn_decode with the library's static device workspace (no allocation)."""
    batch, max_len = K.shape[0], K.shape[2]
    _check("cobs_sparse_attn_decode_static", lib().cobs_sparse_attn_decode_static(
        ctypes.byref(p), batch, max_len, _ptr(seq_lens), _ptr(Q), _ptr(K), _ptr(V), _ptr(mu), _ptr(so),
        _ptr(kc), _ptr(vc), _ptr(gates), _ptr(sel_in), _ptr(sel_out), _ptr(out), _stream(stream)))


def cobs_set_poll_limit(polls: int) -> None:
    """Test hook: polls of a published selection code before a wave gives up."""
    lib().cobs_set_poll_limit(polls & 0xFFFFFFFF)


def cobs_sparse_attn_prefill(p: cobs_params, q_pos0: int, Q, K, V, mu, so, kc, vc, gates, out, ws,
                             sel_out=None, stream=None) -> None:
    seq_len, tokens = K.shape[1], Q.shape[0]
    _check("cobs_sparse_attn_prefill", lib().cobs_sparse_attn_prefill(
        ctypes.byref(p), seq_len, tokens, q_pos0, _ptr(Q), _ptr(K), _ptr(V), _ptr(mu), _ptr(so), _ptr(kc),
        _ptr(vc), _ptr(gates), _ptr(sel_out), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


# ---------------------------------------------------------------------------
# allocation helpers (device memory via torch; plumbing only)
# ---------------------------------------------------------------------------

def alloc_summaries(p: cobs_params, batch: int, max_len: int, device="cuda") -> dict:
    sh = cobs_summary_shapes(p, batch, max_len)
    nb, nc, d, hkv = sh["nb_max"], sh["nc_max"], p.head_dim, p.n_kv_heads
    if p.so_kind == COBS_SO_LOWRANK_FP4:
        # bf16 means; one byte record per block (codes, exponents, padding)
        mu = torch.empty((batch, hkv, nb, d), dtype=torch.bfloat16, device=device)
        so = torch.empty((batch, hkv, nb, sh["so_bytes"] // (batch * hkv * nb)), dtype=torch.uint8, device=device)
    else:
        mu = torch.empty((batch, hkv, nb, d), dtype=torch.float32, device=device)
        vlen = -(-p.subspace_dim // 32) * 32 if p.subspace_dim > 0 else d
        so_shape = (batch, hkv, nb, p.rank, vlen) if p.so_kind == COBS_SO_LOWRANK else (batch, hkv, nb, d)
        so = torch.empty(so_shape, dtype=torch.float32, device=device)
    kdt = torch.bfloat16 if p.kv_dtype == COBS_BF16 else torch.float32
    kc = vc = None
    if nc > 0:
        kc = torch.empty((batch, hkv, nc, d), dtype=kdt, device=device)
        vc = torch.empty((batch, hkv, nc, d), dtype=kdt, device=device)
    return {"mu": mu, "so": so, "kc": kc, "vc": vc, "nb_max": nb, "nc_max": nc}


def cobs_query_subspace(p: cobs_params, Q: torch.Tensor, s: int, stream=None) -> torch.Tensor:
    """Query subspace [H_kv][s][d] (fp32) from calibration queries Q [n][H_q][d]."""
    q = cobs_params.from_buffer_copy(p)
    q.subspace_dim = s
    n = lib().cobs_query_subspace_workspace_bytes(ctypes.byref(q))
    if n == 0:
        raise CobsError("cobs_query_subspace_workspace_bytes", COBS_ERR_INVALID_ARG)
    ws = torch.empty(n, dtype=torch.uint8, device=Q.device)
    P = torch.empty((p.n_kv_heads, s, p.head_dim), dtype=torch.float32, device=Q.device)
    _check("cobs_query_subspace", lib().cobs_query_subspace(ctypes.byref(q), Q.shape[0], _ptr(Q), _ptr(P), _ptr(ws),
                                                            n, _stream(stream)))
    return P


def alloc_workspace(p: cobs_params, batch: int, max_len: int, n_q_tokens: int = 1, device="cuda") -> torch.Tensor:
    n = cobs_workspace_bytes(p, batch, max_len, n_q_tokens)
    if n == 0:
        raise CobsError("cobs_workspace_bytes", COBS_ERR_INVALID_ARG)
    return torch.zeros(n, dtype=torch.uint8, device=device)
