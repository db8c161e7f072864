"""GPU parity of chunked causal prefill against the fp64 oracle.

Each query token t sees the blocks whose keys all lie at positions <= t, the
window [t-W+1, t] and the pooled tokens with 16j+31 <= t; the bars are those of
decode (selection by the 1e-3 score-gap rule, outputs max-abs 1e-2)."""
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


def check_prefill(w, x, tokens, out_tol=1e-2):
    g = U.to_device(x)
    p = U.params_for(w, P=g.get("P"))
    s = U.build(p, g)
    out, sel = U.prefill(p, g, s, w.q_pos0)
    ref = O.run(x, O.params_of(w), tokens=tokens)
    G = w.group
    worst = 0.0
    for (b, h, i), (o_out, o_sel, shat, gap) in ref.items():
        ok, msg = U.selection_ok(sel[i, h], shat, w.top_k)
        assert ok, f"token {i} (t={w.q_pos0 + i}) group {h}: {msg}; gpu {sel[i, h]} oracle {o_sel} gap {gap:.3g}"
        if gap >= U.GAP:
            np.testing.assert_array_equal(sel[i, h], o_sel)
            err = float(np.abs(out[i, h * G:(h + 1) * G] - o_out).max())
            worst = max(worst, err)
            assert err <= out_tol, f"token {i} group {h}: max-abs {err}"
    return worst, out, sel


BASE = dict(batch=1, n_q_heads=32, n_kv_heads=2, head_dim=128, top_k=8, window=300, cmp_len=32, cmp_stride=16,
            so_kind="diag", rank=0, alpha=1.0, dtype="bf16", needles=3)


@pytest.mark.parametrize("T", [200, 37])
def test_prefill_ragged_tail(T):
    """Chunks that are not a multiple of the attention kernel's 16 tokens per
    workgroup (37 = 2 x 16 + 5) nor of the scoring kernel's two (odd)."""
    L = 1500
    w = synth.Workload("pf", max_len=L, min_len=L, n_q_tokens=T, q_pos0=L - T, **BASE)
    x = synth.make_inputs(w, 11)
    check_prefill(w, x, tokens=list(range(T)))


def test_prefill_from_position_zero():
    """Early tokens have no complete block yet (empty selection) but see the
    window and, from t = 31 on, pooled tokens."""
    L, T = 700, 150
    w = synth.Workload("pf0", max_len=L, min_len=L, n_q_tokens=T, q_pos0=0, **dict(BASE, top_k=4))
    x = synth.make_inputs(w, 12)
    worst, out, sel = check_prefill(w, x, tokens=list(range(T)))
    assert (sel[:63] == -1).all()


@pytest.mark.parametrize("kind,d,G", [("lowrank", 128, 4), ("diag", 64, 8)])
def test_prefill_variants(kind, d, G):
    L, T = 900, 64
    w = synth.Workload("pfv", max_len=L, min_len=L, n_q_tokens=T, q_pos0=L - T,
                       **dict(BASE, head_dim=d, n_q_heads=2 * G, so_kind=kind, rank=4 if kind == "lowrank" else 0))
    x = synth.make_inputs(w, 13)
    check_prefill(w, x, tokens=list(range(T)))


def test_prefill_max_top_k():
    """top-k 64 over 78 blocks: the selected-block union of a 16-token workgroup
    covers most of the prefix."""
    L, T = 5000, 40
    w = synth.Workload("pfk", max_len=L, min_len=L, n_q_tokens=T, q_pos0=L - T, **dict(BASE, top_k=64))
    x = synth.make_inputs(w, 17)
    check_prefill(w, x, tokens=list(range(T)))


def test_prefill_f32_inputs():
    # fp32 Q/K/V take the one-workgroup-per-(token, group) attention path
    L, T = 700, 40
    w = synth.Workload("pff", max_len=L, min_len=L, n_q_tokens=T, q_pos0=L - T,
                       **dict(BASE, head_dim=64, n_q_heads=8, dtype="f32", top_k=4, window=100))
    x = synth.make_inputs(w, 16)
    worst, _, _ = check_prefill(w, x, tokens=list(range(T)), out_tol=1e-4)
    assert worst <= 1e-4


def test_prefill_last_token_matches_decode():
    L = 1280
    wp = synth.Workload("pfd", max_len=L, min_len=L, n_q_tokens=1, q_pos0=L - 1, **BASE)
    x = synth.make_inputs(wp, 14)
    p = U.params_for(wp)
    g = U.to_device(x)
    s = U.build(p, g)
    out_p, sel_p = U.prefill(p, g, s, L - 1)
    wd = synth.Workload("pfd", max_len=L, min_len=L, **BASE)
    gd = U.to_device(dict(x, workload=wd))
    out_d, sel_d = U.decode(p, gd, s)
    np.testing.assert_array_equal(sel_p[0], sel_d[0])
    # same keys, different tile split: P is rounded to bf16 against different running
    # maxima, so the two paths agree to the bf16 rounding of the weights (2^-9 relative)
    assert np.abs(out_p[0] - out_d[0]).max() <= 2e-3


def test_select_topk_at_positions_batched():
    w = synth.Workload("pfs", max_len=2000, min_len=1200, n_q_tokens=6, q_pos0=1100, **dict(BASE, batch=2))
    x = synth.make_inputs(w, 15, lens=np.array([2000, 1200]))
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    q = torch.from_numpy(x["Q"]).cuda().to(torch.bfloat16).contiguous()          # [B][T][Hq][d]
    ws = B.alloc_workspace(p, w.batch, w.max_len, w.n_q_tokens)
    sel = torch.full((w.batch, w.n_q_tokens, w.n_kv_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
    score = torch.empty((w.batch, w.n_q_tokens, w.n_kv_heads, s["nb_max"]), dtype=torch.float32, device="cuda")
    B.cobs_select_topk(p, g["lens"], q, s["mu"], s["so"], sel, ws, sel_score=score, max_len=w.max_len,
                       q_pos0=w.q_pos0)
    sel = sel.cpu().numpy()
    score = score.cpu().numpy()
    ref = O.run(x, O.params_of(w))
    for (b, h, i), (o_out, o_sel, shat, gap) in ref.items():
        ok, msg = U.selection_ok(sel[b, i, h], shat, w.top_k)
        assert ok, f"seq {b} token {i} group {h}: {msg}"
        np.testing.assert_allclose(score[b, i, h, :len(shat)], shat, atol=1e-4)
        assert np.isneginf(score[b, i, h, len(shat):]).all()


def test_full_size_prefill_sampled():
    """8192 queries over a 32k prefix: every 16th token (a strided 1/16 of the chunk,
    starting with the first) and the last."""
    w = synth.WORKLOADS["prefill_T8k_L32k"]
    x = synth.make_inputs(w, 3)
    toks = sorted(set(range(0, w.n_q_tokens, 16)) | {w.n_q_tokens - 1})
    check_prefill(w, x, tokens=toks)


def test_prefill_diag_beyond_512_blocks():
    """Diagonal summaries over 625 candidate blocks: the one-workgroup-per-(token,
    group) selection kernel (the two-token kernel covers up to 512 blocks)."""
    L, T = 40000, 40
    w = synth.Workload("pf625", max_len=L, min_len=L, n_q_tokens=T, q_pos0=L - T, **dict(BASE, top_k=16))
    x = synth.make_inputs(w, 18)
    check_prefill(w, x, tokens=list(range(T)))


def test_prefill_beyond_2048_blocks():
    """A 150k-key prefix (2344 blocks): the one-wave-per-(token, group) selection
    kernel for contexts beyond the LDS of the workgroup kernels."""
    L, T = 150000, 24
    w = synth.Workload("pf150k", max_len=L, min_len=L, n_q_tokens=T, q_pos0=L - T,
                       **dict(BASE, n_q_heads=8, n_kv_heads=1, top_k=16, window=512))
    x = synth.make_inputs(w, 19)
    check_prefill(w, x, tokens=list(range(T)))
