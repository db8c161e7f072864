"""The bounded wait of the selected-branch workgroups: a wave that gives up is
reported through cobs_decode_status, every kernel still ends normally, and the next
step on the same workspace is unaffected (no stale selection codes).  The give-up is
forced from the host with the test hook cobs_set_poll_limit(0)."""
import numpy as np
import pytest
import torch

from block_sparse_long_compressed_amd import binding as B
from block_sparse_long_compressed_amd import synth
from oracle import cobs_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _step(p, g, s, ws):
    batch = g["K"].shape[0]
    out = torch.full((batch, p.n_q_heads, p.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((batch, p.n_kv_heads, p.top_k), -7, dtype=torch.int32, device="cuda")
    B.cobs_sparse_attn_decode(p, g["lens"], g["Q"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"], g["gates"],
                              out, ws, sel_out=sel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy()


def test_wait_give_up_is_reported_and_harmless():
    torch.cuda.set_device(0)
    # top-k 32 with 8 units: the selecting workgroup attends to the first few selected
    # blocks and waiting workgroups take the rest
    w = synth.Workload("status_b2_L3000", batch=2, max_len=3000, min_len=2200, n_q_heads=64, n_kv_heads=4,
                       head_dim=128, top_k=32, window=256, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0,
                       alpha=1.0, dtype="bf16", needles=2)
    x = synth.make_inputs(w, 11)
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    ws = B.alloc_workspace(p, w.batch, w.max_len)
    try:
        print("status case: normal step", flush=True)
        out0, sel0 = _step(p, g, s, ws)
        assert B.cobs_decode_status(p, w.batch, w.max_len, ws) == 0
        ref = O.run(x, O.params_of(w))
        G = w.group
        for (b, h, _), (o_out, o_sel, shat, gap) in ref.items():
            ok, msg = U.selection_ok(sel0[b, h], shat, w.top_k)
            assert ok, f"seq {b} group {h}: {msg}"
            if gap >= U.GAP:
                assert float(np.abs(out0[b, h * G:(h + 1) * G] - o_out).max()) <= 1e-2
        print("status case: waits forced to give up", flush=True)
        B.cobs_set_poll_limit(0)
        out1, sel1 = _step(p, g, s, ws)          # every kernel must still end
        assert B.cobs_decode_status(p, w.batch, w.max_len, ws) & B.COBS_STATUS_WAIT_GAVE_UP
        assert B.cobs_decode_status(p, w.batch, w.max_len, ws) == 0      # the query cleared it
        assert np.array_equal(sel1, sel0)        # the selection itself is unaffected
    finally:
        B.cobs_set_poll_limit(0xFFFFFFFF)
    print("status case: next step on the same workspace", flush=True)
    out2, sel2 = _step(p, g, s, ws)
    assert B.cobs_decode_status(p, w.batch, w.max_len, ws) == 0
    assert np.array_equal(sel2, sel0)
    assert np.array_equal(out2, out0), float(np.nanmax(np.abs(out2 - out0)))
