"""GPU selection by exact attention mass (the selection oracle of COBS 2.1, kept as a
quality diagnostic) against the fp64 oracle: the same selection bar as COBS itself
(bit-exact unless the score gap is below 1e-3; group scores to 1e-4), and the recall
of the cumulant selections (alpha = 1 and alpha = 0) measured against it."""
import numpy as np
import pytest
import torch

from block_sparse_long_compressed_amd import binding as B
from block_sparse_long_compressed_amd import synth
from oracle import cobs_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    yield


def exact_select(w, x, g):
    p = U.params_for(w)
    ws = B.alloc_workspace(p, w.batch, w.max_len)
    sel = torch.full((w.batch, w.n_kv_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
    nb = -(-w.max_len // 64)
    score = torch.empty((w.batch, w.n_kv_heads, nb), dtype=torch.float32, device="cuda")
    B.cobs_select_topk_exact(p, g["lens"], g["Q"], g["K"], sel, ws, sel_score=score)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("name,d,G,lens", [
    ("osa-a", 128, 16, [2000, 1234]),
    ("osa-b", 64, 8, [777, 4096]),
])
def test_exact_selection_matches_oracle(name, d, G, lens):
    w = synth.Workload(name, batch=2, max_len=max(lens), min_len=min(lens), n_q_heads=2 * G, n_kv_heads=2,
                       head_dim=d, top_k=8, window=0, cmp_len=0, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0,
                       dtype="bf16", needles=3)
    x = synth.make_inputs(w, 5, lens=np.array(lens))
    g = U.to_device(x)
    sel, score = exact_select(w, x, g)
    op = O.params_of(w)
    for b in range(w.batch):
        L = int(lens[b])
        for h in range(w.n_kv_heads):
            keys = x["K"][b, h, :L].astype(np.float64)
            qg = x["Q"][b, 0, h * G:(h + 1) * G].astype(np.float64)
            cand, shat = O.exact_group_scores(op, qg, keys, L, L - 1)
            ok, msg = U.selection_ok(sel[b, h], shat, w.top_k)
            assert ok, f"seq {b} group {h}: {msg}"
            np.testing.assert_allclose(score[b, h, :len(shat)], shat, atol=1e-4)
            assert np.isneginf(score[b, h, len(shat):]).all()


def test_recall_of_cumulant_selection_against_exact():
    """The measurement the diagnostic exists for: the share of the exact top-k that the
    cumulant selection keeps.  On the needle workload the second-order term must not
    lose recall against the first-order (alpha = 0) selector."""
    w = synth.WORKLOADS["decode_b1_L32k"]
    x = synth.make_inputs(w, 7)
    g = U.to_device(x)
    exact, _ = exact_select(w, x, g)
    rec = {}
    for alpha in (0.0, 1.0):
        p = U.params_for(w, alpha=alpha)
        s = U.build(p, g)
        _, sel = U.decode(p, g, s)
        hit = sum(len(set(sel[b, h][sel[b, h] >= 0]) & set(exact[b, h][exact[b, h] >= 0]))
                  for b in range(w.batch) for h in range(w.n_kv_heads))
        rec[alpha] = hit / (w.batch * w.n_kv_heads * w.top_k)
    print("recall vs exact-mass selection:", rec)
    assert rec[1.0] >= rec[0.0]
    assert rec[1.0] >= 0.5
