"""GPU parity of the query-subspace projection (COBS Technisches Resuemee 2.3,
"Subraum-Projektion") against the fp64 oracle.

- Calibration: the subspace computed on the GPU from calibration queries spans
  the oracle's (projectors P^T P agree to 1e-5 where the s-th eigengap is at
  least 1e-3 relative), and each row whose eigenvalue is separated from both
  neighbours by 1e-3 relative equals the oracle's row to 1e-5 (fp32 output).
- Summaries: with the same (seeded, orthonormal) P on both sides, the rank-r
  approximant of P C P^T agrees to 1e-4 (relative Frobenius) where the eigengap
  is at least 1e-2; the stored vectors are zero beyond s.  For the compressed
  storage the checks of the FP4 tests apply to the padded vectors.
- Selection and outputs: the decode / prefill bars (1e-3 score-gap rule; outputs
  max-abs 1e-2), the oracle scoring with the same P."""
import numpy as np
import pytest
import torch

from block_sparse_long_compressed_amd import binding as B
from block_sparse_long_compressed_amd import synth
from oracle import cobs_oracle as O
from tests import gpu_util as U
from tests.test_gpu_fp4 import check_fp4
from tests.test_gpu_parity import run_and_check
from tests.test_gpu_prefill import check_prefill
from tests.test_gpu_update import run_update, untouched_equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    yield


SUB = dict(batch=2, max_len=1500, min_len=700, n_q_heads=8, n_kv_heads=2, head_dim=128, top_k=6,
           window=200, cmp_len=32, cmp_stride=16, so_kind="lowrank", rank=4, alpha=1.0, dtype="bf16",
           needles=2, subspace=40)


def check_sub_fp32(w, x, s, gap_min=1e-2):
    vlen = -(-w.subspace // 32) * 32
    so_all = s["so"].cpu().numpy()          # blocks past a sequence's end are never written
    mu = s["mu"].cpu().numpy()
    assert so_all.shape[-1] == vlen
    checked = 0
    for b in range(w.batch):
        L = int(x["lens"][b])
        nb_b = -(-L // 64)
        so = {b: so_all[b, :, :nb_b].astype(np.float64)}
        assert np.isfinite(so[b]).all()
        for h in range(w.n_kv_heads):
            keys = x["K"][b, h, :L].astype(np.float64)
            Ph = x["P"][h].astype(np.float64)
            rmu, rso, n = O.summaries(keys, L, "lowrank", w.rank, Ph)
            assert U.rel_err_rows(mu[b, h, :len(n)], rmu) <= 1e-4
            assert (so[b][h, :len(n), :, w.subspace:] == 0).all()
            for blk in range(len(n)):
                C = Ph @ O.block_covariance(keys[blk * 64: blk * 64 + n[blk]]) @ Ph.T
                lam = np.sort(np.linalg.eigvalsh(C))[::-1]
                if n[blk] > w.rank + 1 and (lam[w.rank - 1] - lam[w.rank]) >= gap_min * lam[w.rank - 1]:
                    got = so[b][h, blk, :, :w.subspace]
                    ref = rso[blk].T @ rso[blk]
                    assert np.linalg.norm(got.T @ got - ref) <= 1e-4 * np.linalg.norm(ref), (b, h, blk)
                    checked += 1
    assert checked > 0


@pytest.mark.parametrize("d,s", [(128, 85), (64, 20)])
def test_query_subspace_matches_oracle(d, s):
    w = synth.Workload("cal", **dict(SUB, head_dim=d, subspace=s, n_q_heads=8 if d == 128 else 16))
    x = synth.make_inputs(w, 41, lens=np.array([700, 700]))
    g = U.to_device(x)
    p = U.params_for(w)
    P = B.cobs_query_subspace(p, g["Qcal"], s)
    torch.cuda.synchronize()
    P = P.cpu().numpy().astype(np.float64)
    G = w.group
    rows_checked = 0
    for h in range(w.n_kv_heads):
        qs = x["Qcal"][:, h * G:(h + 1) * G].reshape(-1, d).astype(np.float64)
        ref = O.query_subspace(qs, s)
        lam = np.sort(np.linalg.eigvalsh(qs.T @ qs / qs.shape[0]))[::-1]
        if lam[s - 1] - lam[s] >= 1e-3 * lam[s - 1]:
            assert np.linalg.norm(P[h].T @ P[h] - ref.T @ ref) <= 1e-5 * np.sqrt(s), h
        for i in range(s):
            lo = lam[i] - lam[i + 1] if i + 1 < d else np.inf
            hi = lam[i - 1] - lam[i] if i > 0 else np.inf
            if min(lo, hi) >= 1e-3 * lam[i]:
                np.testing.assert_allclose(P[h, i], ref[i], atol=1e-5)
                rows_checked += 1
    assert rows_checked > 0


@pytest.mark.parametrize("kind,d,s", [("lowrank", 128, 40), ("lowrank", 128, 85), ("lowrank", 64, 20),
                                      ("lowrank_fp4", 128, 85), ("lowrank_fp4", 64, 64)])
def test_summaries_subspace(kind, d, s):
    w = synth.Workload("sub", **dict(SUB, so_kind=kind, head_dim=d, subspace=s, n_q_heads=8 if d == 128 else 16))
    x = synth.make_inputs(w, 42, lens=np.array([1500, 700]))
    g = U.to_device(x)
    p = U.params_for(w, P=g["P"])
    sm = U.build(p, g)
    if kind == "lowrank":
        check_sub_fp32(w, x, sm)
    else:
        check_fp4(w, x, sm)


@pytest.mark.parametrize("kind,alpha", [("lowrank", 1.0), ("lowrank_fp4", 1.0), ("lowrank_fp4", 2.0)])
def test_decode_subspace(kind, alpha):
    w = synth.Workload("sub", **dict(SUB, so_kind=kind, subspace=85))
    x = synth.make_inputs(w, 43, lens=np.array([1500, 777]))
    run_and_check(w, x, alpha=alpha)


def test_decode_subspace_f32_d64():
    w = synth.Workload("sub", **dict(SUB, head_dim=64, n_q_heads=16, dtype="f32", rank=3, subspace=33))
    x = synth.make_inputs(w, 44, lens=np.array([1300, 640]))
    run_and_check(w, x)


def test_prefill_subspace():
    L, T = 900, 64
    w = synth.Workload("pfs", **dict(SUB, so_kind="lowrank_fp4", batch=1, max_len=L, min_len=L, n_q_heads=16,
                                     n_q_tokens=T, q_pos0=L - T, subspace=85))
    x = synth.make_inputs(w, 45)
    check_prefill(w, x, tokens=list(range(T)))


def test_update_subspace():
    w = synth.Workload("upds", **dict(SUB, so_kind="lowrank_fp4", max_len=1100, min_len=500, subspace=85))
    old_lens, new_lens = [1000, 511], [1090, 513]
    x, s, before = run_update(w, new_lens, old_lens, 90)
    check_fp4(w, x, s)
    untouched_equal(s, before, old_lens, w)


def test_full_size_long_decode_subspace():
    """8 x 128k, subspace 85, compressed storage (the paper's headline configuration):
    compressed summaries of 4 units, selections of 16 units over all 8 sequences and
    every kv head, outputs where the gap is unambiguous."""
    from tests.conftest import LONG_UNITS
    from tests.test_gpu_parity import check_long_units
    w = synth.WORKLOADS["decode_b8_L128k_sub85_fp4"]
    x = synth.make_inputs(w, 4)
    g = U.to_device(x)
    p = U.params_for(w, P=g["P"])
    s = U.build(p, g)
    check_fp4(w, x, s, units=[(0, 0), (3, 1), (7, 5), (5, 3)])
    out, sel = U.decode(p, g, s)
    op = O.params_of(w)
    units = {}
    for (b, h) in LONG_UNITS:
        print(f"[test] oracle subspace summaries of unit ({b}, {h})", flush=True)
        L = int(x["lens"][b])
        ph = dict(op, P=x["P"][h].astype(np.float64))
        units[(b, h)] = O.build_unit(ph, x["K"][b, h, :L].astype(np.float64), x["V"][b, h, :L].astype(np.float64), L)
    for (b, h), u in units.items():          # each unit scores with its own kv head's subspace
        check_long_units(w, x, out, sel, {(b, h): u}, dict(op, P=x["P"][h].astype(np.float64)))
