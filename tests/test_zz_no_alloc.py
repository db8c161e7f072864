"""The decode entry point that allocates nothing (cobs_sparse_attn_decode_static)
against cobs_sparse_attn_decode with a caller workspace: two calls in a row on the
library's static array, the second with a smaller batch and shorter context."""
import numpy as np
import pytest
import torch

from block_sparse_long_compressed_amd import binding as B
from block_sparse_long_compressed_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = [  # (batch, max_len, min_len, top_k): the second is smaller than the first
    (4, 6000, 2500, 32),
    (2, 2000, 900, 16),
]


def _case(batch, max_len, min_len, top_k, seed):
    w = synth.Workload(f"noalloc_b{batch}_L{max_len}", batch=batch, max_len=max_len, min_len=min_len, n_q_heads=32,
                       n_kv_heads=2, head_dim=128, top_k=top_k, window=256, cmp_len=32, cmp_stride=16,
                       so_kind="diag", rank=0, alpha=1.0, dtype="bf16", needles=2)
    x = synth.make_inputs(w, seed)
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    return w, p, g, s


def test_static_decode_matches_workspace_decode_twice():
    torch.cuda.set_device(0)
    for i, (batch, max_len, min_len, top_k) in enumerate(CASES):
        print(f"no-alloc case {i}: batch {batch} max_len {max_len} top_k {top_k}", flush=True)
        w, p, g, s = _case(batch, max_len, min_len, top_k, 40 + i)
        out_ref, sel_ref = U.decode(p, g, s)
        out = torch.full((batch, p.n_q_heads, p.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        sel = torch.full((batch, p.n_kv_heads, p.top_k), -7, dtype=torch.int32, device="cuda")
        B.cobs_sparse_attn_decode_static(p, g["lens"], g["Q"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"],
                                         g["gates"], out, sel_out=sel)
        torch.cuda.synchronize()
        o, sl = out.cpu().numpy(), sel.cpu().numpy()
        assert np.array_equal(sl, sel_ref), f"case {i}: selections differ"
        assert np.isfinite(o).all()
        err = float(np.abs(o - out_ref).max())
        assert err <= 1e-6, f"case {i}: outputs differ by {err}"
        assert B.cobs_decode_status(p, batch, max_len, None) == 0
