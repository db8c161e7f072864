"""Shared helpers of the GPU parity tests: move a synthetic batch to the GPU, run
the C-ABI entry points, and check results against the oracle."""
from __future__ import annotations

import numpy as np
import torch

from block_sparse_long_compressed_amd import binding as B

GAP = 1e-3          # score gap (natural-log units) below which several selections are correct
SO_KINDS = {"diag": B.COBS_SO_DIAG, "lowrank": B.COBS_SO_LOWRANK, "lowrank_fp4": B.COBS_SO_LOWRANK_FP4}


def params_for(w, alpha=None, top_k=None, P=None):
    """Parameters of a workload; P (device [H_kv][s][d] fp32) for the subspace kinds."""
    return B.make_params(w.head_dim, w.n_q_heads, w.n_kv_heads, w.top_k if top_k is None else top_k,
                         window=w.window, cmp_len=w.cmp_len, cmp_stride=w.cmp_stride,
                         so_kind=SO_KINDS[w.so_kind],
                         rank=0 if w.so_kind == "diag" else w.rank,
                         alpha=w.alpha if alpha is None else alpha,
                         kv_dtype=B.COBS_BF16 if w.dtype == "bf16" else B.COBS_F32, subspace=P)


def to_device(x: dict, dev="cuda") -> dict:
    w = x["workload"]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = {"K": torch.from_numpy(x["K"]).to(dev).to(dt).contiguous(),
         "V": torch.from_numpy(x["V"]).to(dev).to(dt).contiguous(),
         "lens": torch.from_numpy(x["lens"]).to(dev).contiguous()}
    if x.get("P") is not None:                 # query subspaces (an input of the subspace kinds)
        g["P"] = torch.from_numpy(x["P"]).to(dev).contiguous()
        g["Qcal"] = torch.from_numpy(x["Qcal"]).to(dev).to(dt).contiguous()
    q = torch.from_numpy(x["Q"]).to(dev).to(dt)
    if w.prefill:                      # one sequence: Q [T][Hq][d], gates [T][Hq][3]
        g["Q"] = q[0].contiguous()
        g["gates"] = None if x["gates"] is None else torch.from_numpy(x["gates"][0]).to(dev).contiguous()
    else:                              # decode: Q [B][Hq][d], gates [B][Hq][3]
        g["Q"] = q[:, 0].contiguous()
        g["gates"] = None if x["gates"] is None else torch.from_numpy(x["gates"][:, 0]).to(dev).contiguous()
    return g


def build(p, g) -> dict:
    batch, max_len = g["K"].shape[0], g["K"].shape[2]
    s = B.alloc_summaries(p, batch, max_len)
    B.cobs_build_summaries(p, g["lens"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"])
    return s


def decode(p, g, s, sel_in=None):
    batch, max_len = g["K"].shape[0], g["K"].shape[2]
    ws = B.alloc_workspace(p, batch, max_len)
    out = torch.empty((batch, p.n_q_heads, p.head_dim), dtype=torch.float32, device="cuda")
    sel = torch.full((batch, p.n_kv_heads, p.top_k), -7, dtype=torch.int32, device="cuda")
    B.cobs_sparse_attn_decode(p, g["lens"], g["Q"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"],
                              g["gates"], out, ws, sel_in=sel_in, sel_out=sel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy()


def prefill(p, g, s, q_pos0):
    T = g["Q"].shape[0]
    K0, V0 = g["K"][0].contiguous(), g["V"][0].contiguous()
    kc = None if s["kc"] is None else s["kc"][0].contiguous()
    vc = None if s["vc"] is None else s["vc"][0].contiguous()
    ws = B.alloc_workspace(p, 1, K0.shape[1], T)
    out = torch.empty((T, p.n_q_heads, p.head_dim), dtype=torch.float32, device="cuda")
    sel = torch.full((T, p.n_kv_heads, p.top_k), -7, dtype=torch.int32, device="cuda")
    B.cobs_sparse_attn_prefill(p, q_pos0, g["Q"], K0, V0, s["mu"], s["so"], kc, vc, g["gates"], out, ws,
                               sel_out=sel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy()


def selection_ok(sel_gpu: np.ndarray, shat: np.ndarray, k: int, cand_offset: int = 0):
    """Is the GPU selection one of the correct top-k sets of the oracle scores shat
    (over candidate blocks 0..len(shat)-1)?  Returns (ok, message)."""
    nc = len(shat)
    take = min(k, nc)
    chosen = [int(b) for b in sel_gpu if b >= 0]
    if list(sel_gpu[take:]) != [-1] * (k - take):
        return False, f"padding wrong: {sel_gpu}"
    if len(chosen) != take or chosen != sorted(chosen) or len(set(chosen)) != take:
        return False, f"not {take} ascending distinct blocks: {sel_gpu}"
    if take == 0:
        return True, ""
    if max(chosen) >= nc:
        return False, f"non-candidate selected: {chosen} (candidates {nc})"
    order = sorted(range(nc), key=lambda b: (-shat[b], b))
    sk = shat[order[take - 1]]
    sk1 = shat[order[take]] if take < nc else -np.inf
    sure_in = {b for b in range(nc) if shat[b] - sk1 >= GAP}
    sure_out = {b for b in range(nc) if sk - shat[b] >= GAP}
    S = set(chosen)
    if not sure_in <= S:
        return False, f"missing sure blocks {sorted(sure_in - S)}"
    if S & sure_out:
        return False, f"selected excluded blocks {sorted(S & sure_out)}"
    return True, ""


def rel_err_rows(a: np.ndarray, b: np.ndarray) -> float:
    """Largest per-row relative L2 error of a against reference b."""
    num = np.linalg.norm(a - b, axis=-1)
    den = np.maximum(np.linalg.norm(b, axis=-1), 1e-30)
    return float((num / den).max())


def bf16_round64(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of fp64 values, returned as fp64."""
    f = x.astype(np.float32)
    # fp64 -> fp32 rounding first cannot create a double rounding error large enough to
    # matter at the +-1 ulp bar used by the callers
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)
