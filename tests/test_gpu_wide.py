"""Decode with the eight-wave plan (one scoring workgroup per unit, block scores kept
in LDS, the selecting workgroup attending to its share of the selected blocks) for
every score kind: 64 units and short contexts select that plan.  The batch-32
workload covers it for the diagonal kind at full size; here the rank-r, compressed
and subspace kinds and fp32 keys at d = 64 run it too, against the oracle on a
sample of sequences (selection by the gap rule, outputs where it is unambiguous and
with the oracle's selection everywhere)."""
import numpy as np
import pytest
import torch

from block_sparse_long_compressed_amd import binding as B
from block_sparse_long_compressed_amd import synth
from tests.test_gpu_parity import run_and_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    yield


BASE = dict(batch=16, max_len=2000, min_len=700, n_q_heads=16, n_kv_heads=4, head_dim=128, top_k=8,
            window=200, cmp_len=32, cmp_stride=16, alpha=1.0, dtype="bf16", needles=2)

KINDS = {
    "diag_f32_d64": dict(so_kind="diag", rank=0, dtype="f32", head_dim=64),
    "lowrank": dict(so_kind="lowrank", rank=4),
    "lowrank_fp4": dict(so_kind="lowrank_fp4", rank=4),
    "lowrank_sub": dict(so_kind="lowrank", rank=4, subspace=40),
    "lowrank_fp4_sub": dict(so_kind="lowrank_fp4", rank=4, subspace=40),
}


@pytest.mark.parametrize("kind", list(KINDS))
def test_decode_eight_wave_plan(kind):
    w = synth.Workload(f"wide_{kind}", **dict(BASE, **KINDS[kind]))
    assert w.batch * w.n_kv_heads >= 64
    lens = np.linspace(w.max_len, w.min_len, w.batch).astype(np.int64)
    x = synth.make_inputs(w, 41, lens=lens)
    print(f"[test] eight-wave plan, {kind}", flush=True)
    run_and_check(w, x, seqs=[0, 7, 15])
