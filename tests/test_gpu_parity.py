"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Bars: summaries 1e-4 relative per block; pooled bf16 tokens within 1 ulp of the
rounded oracle mean; selections exactly the oracle's except where the oracle's
k-th / (k+1)-th score gap is below 1e-3 (then any correct top-k set passes);
outputs max-abs 1e-2 on bf16 inputs (1e-4 on fp32 inputs).
"""
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
    B.lib()          # the HIP library must be present: no fallback
    yield


def W(name, **kw):
    return synth.Workload(name, **kw)


SMALL = {
    # several tiles and ragged tails; group 16, window not a multiple of 64
    "g16_d128_bf16": dict(batch=3, max_len=4000, min_len=1111, n_q_heads=32, n_kv_heads=2, head_dim=128,
                          top_k=8, window=300, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0,
                          dtype="bf16", needles=3),
    # fewer blocks than k for a short sequence; window longer than the sequence
    "g4_d128_bf16_short": dict(batch=2, max_len=3000, min_len=130, n_q_heads=8, n_kv_heads=2, head_dim=128,
                               top_k=16, window=1000, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0,
                               alpha=1.0, dtype="bf16", needles=2),
    "g8_d64_bf16": dict(batch=2, max_len=2100, min_len=700, n_q_heads=16, n_kv_heads=2, head_dim=64, top_k=5,
                        window=64, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0, dtype="bf16",
                        needles=2),
    "g2_d64_bf16_nocmp": dict(batch=2, max_len=900, min_len=31, n_q_heads=4, n_kv_heads=2, head_dim=64,
                              top_k=3, window=0, cmp_len=0, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0,
                              dtype="bf16", needles=1),
}


def small(name, seed=1, lens=None):
    w = W(name, **SMALL[name])
    if lens is None:
        lens = {"g16_d128_bf16": [4000, 2500, 1111], "g4_d128_bf16_short": [3000, 130],
                "g8_d64_bf16": [2100, 700], "g2_d64_bf16_nocmp": [900, 31]}[name]
    return w, synth.make_inputs(w, seed, lens=np.array(lens))


def check_summaries(w, x, s):
    p = O.params_of(w)
    mu = s["mu"].cpu().numpy()
    so = s["so"].cpu().numpy()
    kc = None if s["kc"] is None else s["kc"].float().cpu().numpy()
    vc = None if s["vc"] is None else s["vc"].float().cpu().numpy()
    for b in range(w.batch):
        L = int(x["lens"][b])
        for h in range(w.n_kv_heads):
            keys = x["K"][b, h, :L].astype(np.float64)
            vals = x["V"][b, h, :L].astype(np.float64)
            (rmu, rso, n), rkc, rvc = O.build_unit(p, keys, vals, L)
            nb = len(n)
            assert U.rel_err_rows(mu[b, h, :nb], rmu) <= 1e-4, (b, h)
            if w.so_kind == "diag":
                assert U.rel_err_rows(so[b, h, :nb], rso) <= 1e-4, (b, h)
            nc = len(rkc)
            if nc and kc is not None:
                if w.dtype == "bf16":
                    for got, ref in ((kc[b, h, :nc], rkc), (vc[b, h, :nc], rvc)):
                        rr = U.bf16_round64(ref)
                        ulp = np.maximum(np.abs(rr), 1e-38) * 2.0 ** -7
                        assert (np.abs(got - rr) <= ulp * 1.0001).all(), (b, h)
                else:
                    np.testing.assert_allclose(kc[b, h, :nc], rkc, rtol=1e-5, atol=1e-6)
                    np.testing.assert_allclose(vc[b, h, :nc], rvc, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("name", list(SMALL))
def test_summaries_small(name):
    w, x = small(name)
    p = U.params_for(w)
    g = U.to_device(x)
    check_summaries(w, x, U.build(p, g))


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (128, "f32"), (64, "f32")])
def test_summaries_short_and_ragged(d, dtype):
    """Sequences of 1, 31, 33, 64, 65 and 80 keys: a lone partial block, no pooled
    token, a pooled token whose second chunk is the next block's first, and runs of
    blocks that end past the sequence."""
    lens = [1, 31, 33, 64, 65, 80]
    w = W("short", batch=len(lens), max_len=96, min_len=1, n_q_heads=8, n_kv_heads=2, head_dim=d, top_k=2,
          window=64, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0, dtype=dtype, needles=0)
    x = synth.make_inputs(w, 11, lens=np.array(lens))
    p = U.params_for(w)
    check_summaries(w, x, U.build(p, U.to_device(x)))


def test_summaries_tiny_f32():
    w = synth.WORKLOADS["tiny_f32_L1k"]
    x = synth.make_inputs(w, 0)
    p = U.params_for(w)
    check_summaries(w, x, U.build(p, U.to_device(x)))


def run_and_check(w, x, alpha=None, out_tol=1e-2, seqs=None):
    """Full decode on the GPU vs the oracle: selection by the gap rule, outputs
    where the selection is unambiguous, and outputs of the attention path fed with
    the oracle's selection everywhere."""
    g = U.to_device(x)
    p = U.params_for(w, alpha=alpha, P=g.get("P"))
    s = U.build(p, g)
    out, sel = U.decode(p, g, s)
    op = O.params_of(w, alpha=alpha)
    seqs = range(w.batch) if seqs is None else seqs
    ref = O.run(x, op, seqs=seqs)
    G = w.group
    oracle_sel = np.full_like(sel, -1)
    for (b, h, _), (o_out, o_sel, shat, gap) in ref.items():
        ok, msg = U.selection_ok(sel[b, h], shat, w.top_k)
        assert ok, f"seq {b} group {h}: {msg}; gpu {sel[b, h]} oracle {o_sel} gap {gap:.3g}"
        oracle_sel[b, h] = o_sel
        if gap >= U.GAP:
            np.testing.assert_array_equal(sel[b, h], o_sel)
            err = np.abs(out[b, h * G:(h + 1) * G] - o_out).max()
            assert err <= out_tol, f"seq {b} group {h}: max-abs {err}"
    # attention path on the oracle's own selection (covers ambiguous-gap units too)
    sel_in = torch.from_numpy(oracle_sel.astype(np.int32)).cuda()
    for b in range(w.batch):
        if b not in set(seqs):
            sel_in[b] = torch.from_numpy(sel[b].astype(np.int32)).cuda()
    out2, sel2 = U.decode(p, g, s, sel_in=sel_in)
    np.testing.assert_array_equal(sel2, sel_in.cpu().numpy())
    worst = 0.0
    for (b, h, _), (o_out, o_sel, shat, gap) in ref.items():
        err = np.abs(out2[b, h * G:(h + 1) * G] - o_out).max()
        worst = max(worst, err)
        assert err <= out_tol, f"seq {b} group {h}: max-abs {err} with the oracle's selection"
    return worst


@pytest.mark.parametrize("lens", [[5000, 3333], [2000, 700]])
def test_decode_max_top_k(lens):
    """The largest top-k the library accepts (64): most candidates selected at 5000
    keys, all of them (and -1 padding) at 700 keys (11 blocks)."""
    w = W("k64", batch=2, max_len=5000, min_len=700, n_q_heads=32, n_kv_heads=2, head_dim=128, top_k=64,
          window=256, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0, dtype="bf16", needles=3)
    x = synth.make_inputs(w, 21, lens=np.array(lens))
    run_and_check(w, x)


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0, 2.0])
def test_decode_g16_alpha_sweep(alpha):
    w, x = small("g16_d128_bf16")
    run_and_check(w, x, alpha=alpha)


@pytest.mark.parametrize("name", ["g4_d128_bf16_short", "g8_d64_bf16", "g2_d64_bf16_nocmp"])
def test_decode_small(name):
    w, x = small(name)
    run_and_check(w, x)


def test_decode_tiny_f32():
    w = synth.WORKLOADS["tiny_f32_L1k"]
    for seed in range(3):
        x = synth.make_inputs(w, seed)
        worst = run_and_check(w, x, out_tol=1e-4)
        assert worst < 1e-4


def test_decode_f32_d128():
    """fp32 inputs at d = 128 (four-wave workgroups: the attention tile then needs a
    SIMD's whole register file)."""
    w = W("f32d128", batch=2, max_len=2500, min_len=900, n_q_heads=16, n_kv_heads=2, head_dim=128, top_k=8,
          window=200, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0, dtype="f32", needles=2)
    x = synth.make_inputs(w, 23, lens=np.array([2500, 900]))
    worst = run_and_check(w, x, out_tol=1e-4)
    assert worst <= 1e-4


@pytest.mark.parametrize("L", [200000, 262144])
def test_decode_beyond_2048_blocks(L):
    """Contexts of 3125 and 4096 blocks (the most the library accepts): the scoring is
    split over several workgroups whose block scores are handed off through the
    workspace."""
    w = W("long1", batch=1, max_len=L, min_len=L, n_q_heads=8, n_kv_heads=1, head_dim=128, top_k=16,
          window=512, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0, dtype="bf16", needles=4)
    x = synth.make_inputs(w, 24)
    run_and_check(w, x)


def test_decode_single_block_and_tiny_lengths():
    name = "g2_d64_bf16_nocmp"
    w = W(name, **dict(SMALL[name], window=16, max_len=70))
    x = synth.make_inputs(w, 3, lens=np.array([1, 70]))
    run_and_check(w, x)


def test_exact_ties_go_to_lower_block_index():
    name = "g2_d64_bf16_nocmp"
    w = W(name, **dict(SMALL[name], n_q_heads=1, n_kv_heads=1, batch=1, top_k=1, max_len=640, min_len=640))
    x = synth.make_inputs(w, 4)
    q = x["Q"][0, 0, 0].astype(np.float64)
    blk = x["K"][0, 0, 64 * 2: 64 * 3].copy()
    blk[:8] = synth.round_bf16((2.5 * q / np.linalg.norm(q) * 8).astype(np.float32))  # dominant block
    x["K"][0, 0, 64 * 2: 64 * 3] = blk
    x["K"][0, 0, 64 * 7: 64 * 8] = blk                                                # exact duplicate
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    out, sel = U.decode(p, g, s)
    ref = O.run(x, O.params_of(w))[(0, 0, 0)]
    assert ref[2][2] == ref[2][7] and list(ref[1]) == [2]
    assert list(sel[0, 0]) == [2]


def test_decode_is_deterministic():
    w, x = small("g16_d128_bf16")
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    a = U.decode(p, g, s)
    b = U.decode(p, g, s)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_select_topk_scores_match_oracle():
    w, x = small("g16_d128_bf16")
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    nb = s["nb_max"]
    ws = B.alloc_workspace(p, w.batch, w.max_len)
    sel = torch.empty((w.batch, 1, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    score = torch.empty((w.batch, 1, w.n_kv_heads, nb), dtype=torch.float32, device="cuda")
    B.cobs_select_topk(p, g["lens"], g["Q"][:, None].contiguous(), s["mu"], s["so"], sel, ws,
                       sel_score=score, max_len=w.max_len)
    score = score.cpu().numpy()
    ref = O.run(x, O.params_of(w))
    for (b, h, _), (o_out, o_sel, shat, gap) in ref.items():
        ncand = len(shat)
        np.testing.assert_allclose(score[b, 0, h, :ncand], shat, rtol=0, atol=1e-4)
        assert np.isneginf(score[b, 0, h, ncand:]).all()


# ---------------------------------------------------------------------------
# full-size workloads (the configuration the benchmark times), sampled
# ---------------------------------------------------------------------------

def test_full_size_decode_b1_L32k():
    w = synth.WORKLOADS["decode_b1_L32k"]
    x = synth.make_inputs(w, 1)
    run_and_check(w, x)


@pytest.fixture(scope="module")
def batched_inputs():
    w = synth.WORKLOADS["decode_b32_L16k32k"]
    return w, synth.make_inputs(w, 2)


@pytest.fixture(scope="module")
def batched_device(batched_inputs):
    """The batch on the GPU and its summaries (the summaries do not depend on alpha)."""
    w, x = batched_inputs
    g = U.to_device(x)
    s = U.build(U.params_for(w), g)
    return g, s


@pytest.fixture(scope="module")
def batched_oracle(batched_inputs):
    """The oracle's summaries and pooled tokens of every (sequence, kv-head)."""
    w, x = batched_inputs
    p = O.params_of(w)
    units = {}
    for b in range(w.batch):
        L = int(x["lens"][b])
        print(f"[fixture] oracle summaries of sequence {b}", flush=True)
        for h in range(w.n_kv_heads):
            units[(b, h)] = O.build_unit(p, x["K"][b, h, :L].astype(np.float64),
                                         x["V"][b, h, :L].astype(np.float64), L)
    return units


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0, 2.0])
def test_full_size_batched_decode_all_units(alpha, batched_inputs, batched_device, batched_oracle):
    """Batch 32, lengths 16k-32k, in the launch configuration the benchmark times:
    the selection of every (sequence, kv-head) by the gap rule at each alpha; at
    alpha = 1 every output too, where the gap is unambiguous from the fused step and
    everywhere from the attention path fed with the oracle's own selection."""
    w, x = batched_inputs
    g, s = batched_device
    p = U.params_for(w, alpha=alpha)
    out, sel = U.decode(p, g, s)
    op = O.params_of(w, alpha=alpha)
    G = w.group
    oracle_sel = np.full_like(sel, -1)
    oracle_out = {}
    outs = 0
    for b in range(w.batch):
        L = int(x["lens"][b])
        for h in range(w.n_kv_heads):
            summ, kc, vc = batched_oracle[(b, h)]
            qg = x["Q"][b, 0, h * G:(h + 1) * G].astype(np.float64)
            if alpha == 1.0:
                keys = x["K"][b, h, :L].astype(np.float64)
                vals = x["V"][b, h, :L].astype(np.float64)
                gt = x["gates"][b, 0, h * G:(h + 1) * G].astype(np.float64)
                o_out, o_sel, shat, gap = O.query_group(op, qg, keys, vals, L, L - 1, summ, kc, vc, gt)
                oracle_out[(b, h)] = o_out
            else:
                mu, so, n = summ
                shat = O.group_scores(O.block_scores(qg, mu, so, n, alpha, op["scale"], op["so_kind"]))
                o_sel, gap = O.select_topk(shat, w.top_k)
            ok, msg = U.selection_ok(sel[b, h], shat, w.top_k)
            assert ok, f"alpha {alpha} seq {b} group {h}: {msg}; gap {gap:.3g}"
            oracle_sel[b, h] = o_sel
            if gap >= U.GAP:
                np.testing.assert_array_equal(sel[b, h], o_sel)
                if alpha == 1.0:
                    err = float(np.abs(out[b, h * G:(h + 1) * G] - o_out).max())
                    assert err <= 1e-2, f"seq {b} group {h}: max-abs {err}"
                    outs += 1
    if alpha == 1.0:
        assert outs >= w.batch * w.n_kv_heads // 2
        # every unit's outputs on the oracle's selection (attention roles with a given selection)
        sel_in = torch.from_numpy(oracle_sel.astype(np.int32)).cuda()
        out2, _ = U.decode(p, g, s, sel_in=sel_in)
        for (b, h), o_out in oracle_out.items():
            err = float(np.abs(out2[b, h * G:(h + 1) * G] - o_out).max())
            assert err <= 1e-2, f"seq {b} group {h}: max-abs {err} with the oracle's selection"


# ---------------------------------------------------------------------------
# rank-r second-order summaries
# ---------------------------------------------------------------------------

LOWRANK = dict(batch=2, max_len=1500, min_len=700, n_q_heads=8, n_kv_heads=2, head_dim=128, top_k=6,
               window=200, cmp_len=32, cmp_stride=16, so_kind="lowrank", rank=4, alpha=1.0, dtype="bf16",
               needles=2)


def check_lowrank(w, x, s, units=None, gap_min=1e-2):
    """Rank-r approximant sum_i v_i v_i^T against the oracle's, per block.

    Where the oracle's relative eigengap (lambda_r - lambda_r+1)/lambda_r is at least
    gap_min the approximant is well defined and must agree to 1e-4 (relative
    Frobenius); elsewhere the scores it produces for the workload's own queries must
    agree to 1e-4 of the quadratic term's scale."""
    p = O.params_of(w)
    so = s["so"].cpu().numpy()
    mu = s["mu"].cpu().numpy()
    G = w.group
    units = units or [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    checked = loose = 0
    for (b, h) in units:
        print(f"[test] rank-r summaries of unit ({b}, {h})", flush=True)
        L = int(x["lens"][b])
        keys = x["K"][b, h, :L].astype(np.float64)
        rmu, rso, n = O.summaries(keys, L, "lowrank", w.rank)
        assert U.rel_err_rows(mu[b, h, :len(n)], rmu) <= 1e-4
        q = x["Q"][b, 0, h * G:(h + 1) * G].astype(np.float64) * p["scale"]
        for blk in range(len(n)):
            ref = rso[blk].T @ rso[blk]
            got = so[b, h, blk].astype(np.float64).T @ so[b, h, blk].astype(np.float64)
            den = max(np.linalg.norm(ref), 1e-30)
            lam = np.sort(np.linalg.eigvalsh(O.block_covariance(keys[blk * 64: blk * 64 + n[blk]])))[::-1]
            if n[blk] > w.rank + 1 and (lam[w.rank - 1] - lam[w.rank]) >= gap_min * lam[w.rank - 1]:
                assert np.linalg.norm(got - ref) <= 1e-4 * den, (b, h, blk)
                checked += 1
            else:
                qq = np.einsum("hd,de,he->h", q, got - ref, q)
                assert np.abs(qq).max() <= 1e-4 * max(1.0, float(np.abs(np.einsum("hd,de,he->h", q, ref, q)).max())), (b, h, blk)
                loose += 1
    assert checked > 0
    return checked, loose


@pytest.mark.parametrize("rank", [1, 4, 8])
def test_summaries_lowrank(rank):
    w = W("lowrank", **dict(LOWRANK, rank=rank))
    x = synth.make_inputs(w, 5, lens=np.array([1500, 700]))
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    check_lowrank(w, x, s)


def test_summaries_lowrank_repeated_eigenvalues():
    """Blocks whose covariance has an exactly repeated eigenvalue (keys on m
    coordinate axes with equal weight, bf16-exact), a block of identical keys and a
    block whose covariance has rank 2: the rank-4 projector must match the oracle's
    wherever it is well defined, and the quadratic form elsewhere."""
    w = W("lowrank", **dict(LOWRANK, rank=4))
    x = synth.make_inputs(w, 7, lens=np.array([1500, 700]))
    K = x["K"]

    def axes_block(m, a, off):
        blk = np.zeros((64, w.head_dim), dtype=K.dtype)
        for j in range(64):
            blk[j, j % m] = a if (j // m) % 2 == 0 else -a
        return blk + off

    K[0, 0, 64:128] = axes_block(4, 0.75, 0.25)      # four equal eigenvalues, the rest zero
    K[0, 0, 128:192] = axes_block(2, 1.5, 0.0)       # two equal
    K[0, 0, 192:256] = axes_block(3, 0.5, -0.5)      # three equal
    K[0, 0, 256:320] = 0.375                         # identical keys: zero covariance
    K[0, 1, 320:384] = axes_block(4, 1.0, 0.0)
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    checked, loose = check_lowrank(w, x, s)
    assert checked > 0 and loose > 0


@pytest.mark.parametrize("alpha", [0.0, 1.0, 2.0])
def test_decode_lowrank_small(alpha):
    w = W("lowrank", **LOWRANK)
    x = synth.make_inputs(w, 6, lens=np.array([1500, 777]))
    run_and_check(w, x, alpha=alpha)


def check_long_units(w, x, out, sel, oracle_units, p):
    """Selections of the given units by the gap rule and their outputs where the gap
    is unambiguous, from the oracle's summaries of those units."""
    G = w.group
    outs = 0
    for (b, h), (summ, kc, vc) in oracle_units.items():
        print(f"[test] oracle query of unit ({b}, {h})", flush=True)
        L = int(x["lens"][b])
        qg = x["Q"][b, 0, h * G:(h + 1) * G].astype(np.float64)
        gt = x["gates"][b, 0, h * G:(h + 1) * G].astype(np.float64)
        o_out, o_sel, shat, gap = O.query_group(p, qg, x["K"][b, h, :L].astype(np.float64),
                                                x["V"][b, h, :L].astype(np.float64), L, L - 1, summ, kc, vc, gt)
        ok, msg = U.selection_ok(sel[b, h], shat, w.top_k)
        assert ok, f"seq {b} group {h}: {msg}"
        if gap >= U.GAP:
            np.testing.assert_array_equal(sel[b, h], o_sel)
            err = float(np.abs(out[b, h * G:(h + 1) * G] - o_out).max())
            assert err <= 1e-2, f"seq {b} group {h}: max-abs {err}"
            outs += 1
    assert outs >= len(oracle_units) // 2
    return outs


def test_full_size_long_decode_rank4(long_inputs, long_oracle_lowrank):
    """8 x 128k, rank 4 (fp32 storage): selections of 16 units over all 8 sequences and
    every kv head, outputs where the gap is unambiguous, rank-4 summaries of 4 units."""
    w, x = long_inputs
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    check_lowrank(w, x, s, units=[(0, 0), (2, 6), (5, 7), (7, 5)])
    out, sel = U.decode(p, g, s)
    check_long_units(w, x, out, sel, long_oracle_lowrank, O.params_of(w))


def test_decode_graph_replays_match_eager():
    """The benchmark replays captured decode steps; every replay, with eager work and
    synchronisations in between, must reproduce the eager result exactly."""
    w, x = small("g16_d128_bf16")
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    eager_out, eager_sel = U.decode(p, g, s)
    ws = B.alloc_workspace(p, w.batch, w.max_len)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    step = lambda: B.cobs_sparse_attn_decode(p, g["lens"], g["Q"], g["K"], g["V"], s["mu"], s["so"], s["kc"],
                                             s["vc"], g["gates"], out, ws, sel_out=sel)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        sel.fill_(-9)
        scratch = torch.randn(1 << 20, device="cuda").sum()          # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(sel.cpu().numpy(), eager_sel)
        np.testing.assert_array_equal(out.cpu().numpy(), eager_out)
        assert torch.isfinite(scratch)
