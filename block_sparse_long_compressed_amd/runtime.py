"""Device-side conveniences over the C ABI for a synthetic workload: upload a batch,
build its summaries, run one decode step or one prefill chunk.

Argument marshalling and torch allocations only; every step of the method runs in
libcobs.so.  Used by the benchmark and the GPU tests alike.
"""
from __future__ import annotations

import torch

from . import binding as B

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
    """Upload a batch drawn by synth.make_inputs: K, V [B][H_kv][max_len][d], lens, and
    Q / gates in the decode ([B][H_q][..]) or prefill ([T][H_q][..]) layout."""
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
    """Summaries of the uploaded batch (cobs_build_summaries)."""
    batch, max_len = g["K"].shape[0], g["K"].shape[2]
    s = B.alloc_summaries(p, batch, max_len)
    B.cobs_build_summaries(p, g["lens"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"])
    return s


def decode(p, g, s, sel_in=None):
    """One decode step; returns (out [B][H_q][d], sel [B][H_kv][k]) as numpy arrays."""
    batch, max_len = g["K"].shape[0], g["K"].shape[2]
    ws = B.alloc_workspace(p, batch, max_len)
    out = torch.empty((batch, p.n_q_heads, p.head_dim), dtype=torch.float32, device="cuda")
    sel = torch.full((batch, p.n_kv_heads, p.top_k), -7, dtype=torch.int32, device="cuda")
    B.cobs_sparse_attn_decode(p, g["lens"], g["Q"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"],
                              g["gates"], out, ws, sel_in=sel_in, sel_out=sel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy()


def prefill(p, g, s, q_pos0):
    """One prefill chunk of the batch's one sequence; returns (out [T][H_q][d], sel [T][H_kv][k])."""
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
