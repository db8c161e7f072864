"""GPU parity of the incremental summary update (tokens appended to the cache).

After cobs_update_summaries(old_lens -> new_lens) the summaries must be those of
the longer prefix: each block's mean and second-order channel and each complete
pooled token against the fp64 oracle at new_lens (the bars of the summary build:
1e-4 relative; pooled bf16 tokens within one bf16 ulp of the rounded mean), and
every entry the new positions do not touch must be left bit-for-bit as it was."""
import numpy as np
import pytest
import torch

from block_sparse_long_compressed_amd import binding as B
from block_sparse_long_compressed_amd import synth
from tests import gpu_util as U
from tests.test_gpu_parity import check_lowrank, check_summaries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    yield


BASE = dict(n_q_heads=16, n_kv_heads=2, head_dim=128, top_k=8, window=256, cmp_len=32, cmp_stride=16,
            so_kind="diag", rank=0, alpha=1.0, dtype="bf16", needles=2)


def run_update(w, new_lens, old_lens, max_append):
    """Build at old_lens (where > 0), update to new_lens; returns (inputs at new_lens,
    summaries, snapshot of the summaries before the update)."""
    x = synth.make_inputs(w, 21, lens=np.array(new_lens))
    g = U.to_device(x)
    p = U.params_for(w, P=g.get("P"))
    s = B.alloc_summaries(p, w.batch, w.max_len)
    for t in (s["mu"], s["so"], s["kc"], s["vc"]):
        if t is not None:
            # anything the update must write is visibly wrong
            t.fill_(float("nan") if t.is_floating_point() else 0xA5)
    old = torch.tensor(old_lens, dtype=torch.int32, device="cuda")
    new = torch.tensor(new_lens, dtype=torch.int32, device="cuda")
    if min(old_lens) > 0:
        B.cobs_build_summaries(p, old, g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"])
    torch.cuda.synchronize()
    before = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in s.items()}
    B.cobs_update_summaries(p, old, new, max_append, g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"])
    torch.cuda.synchronize()
    return x, s, before


def untouched_equal(s, before, old_lens, w):
    """Blocks wholly below old_len and pooled tokens complete before it are unchanged."""
    for b, L0 in enumerate(old_lens):
        nb_keep = L0 // 64
        nc_keep = (L0 - 32) // 16 + 1 if L0 >= 32 else 0
        for k in ("mu", "so"):
            assert torch.equal(s[k][b, :, :nb_keep], before[k][b, :, :nb_keep]), (k, b)
        if s["kc"] is not None and nc_keep:
            for k in ("kc", "vc"):
                assert torch.equal(s[k][b, :, :nc_keep], before[k][b, :, :nc_keep]), (k, b)


@pytest.mark.parametrize("old_lens,new_lens", [
    ([1000, 2047], [1001, 2048]),       # one token: inside a block / completing a block
    ([1024, 1039], [1025, 1040]),       # first row of a new block / completes pooled token 63
    ([1055, 990], [1056, 991]),         # pooled-token boundary (16j+31 = 1055) / mid-block
])
def test_append_one_token(old_lens, new_lens):
    w = synth.Workload("upd1", batch=2, max_len=2048, min_len=900, **BASE)
    x, s, before = run_update(w, new_lens, old_lens, 1)
    check_summaries(w, x, s)
    untouched_equal(s, before, old_lens, w)


def test_append_many_tokens_ragged():
    # 0..300 new positions per sequence (several blocks and pooled tokens each)
    old_lens, new_lens = [700, 1500, 1999, 64], [1000, 1501, 1999, 364]
    w = synth.Workload("updn", batch=4, max_len=2000, min_len=300, **BASE)
    x, s, before = run_update(w, new_lens, old_lens, 300)
    check_summaries(w, x, s)
    untouched_equal(s, before, old_lens, w)


def test_update_from_empty_equals_build():
    w = synth.Workload("upd0", batch=2, max_len=1500, min_len=1500, **BASE)
    x, s, _ = run_update(w, [1500, 777], [0, 0], 1500)
    check_summaries(w, x, s)


def test_max_append_too_small_still_updates_every_block():
    # max_append only sizes the launch; the workgroups stride over all touched blocks
    old_lens, new_lens = [100, 400], [900, 401]
    w = synth.Workload("upds", batch=2, max_len=1024, min_len=300, **BASE)
    x, s, before = run_update(w, new_lens, old_lens, 1)
    check_summaries(w, x, s)
    untouched_equal(s, before, old_lens, w)


@pytest.mark.parametrize("d,G", [(64, 8)])
def test_append_diag_d64_no_pool(d, G):
    w = synth.Workload("updd", batch=2, max_len=1200, min_len=500, **dict(
        BASE, head_dim=d, n_q_heads=G * 2, cmp_len=0, window=0))
    x, s, before = run_update(w, [1200, 640], [1100, 639], 100)
    assert s["kc"] is None
    check_summaries(w, x, s)
    untouched_equal(s, before, [1100, 639], w)


def test_append_lowrank():
    w = synth.Workload("updr", batch=2, max_len=1100, min_len=500, **dict(BASE, so_kind="lowrank", rank=4))
    old_lens, new_lens = [1000, 511], [1090, 513]
    x, s, before = run_update(w, new_lens, old_lens, 90)
    check_lowrank(w, x, s)
    untouched_equal(s, before, old_lens, w)
