"""GPU parity of the compressed summary storage (COBS Technisches Resuemee 2.3:
bf16 mean, FP4 eigenvectors) against the fp64 oracle.

Summaries: each stored bf16 mean is within one bf16 ulp of the oracle's rounded
fp64 mean (the kernel rounds its fp32 mean), and at least 99% are equal.  Where
the oracle's block has well-separated eigenvalues (the rank-r approximant is then
unique and both sides agree on the vectors to ~1e-10), every FP4 code and every
group exponent equals the oracle's MX quantization of its own vectors, except
entries whose scaled value lies within 1e-6 of a rounding midpoint (and groups
whose maximum lies within 1e-9 of a power of two), where either neighbour is a
correct rounding; those must stay rare.  Elsewhere the dequantized approximant
must give the workload's queries the oracle's quadratic term to 1e-3.

Selection and outputs: the decode and prefill bars of the other kinds (the 1e-3
score-gap rule; outputs max-abs 1e-2), with the oracle scoring its own
compressed summaries."""
import numpy as np
import pytest
import torch

from block_sparse_long_compressed_amd import binding as B
from block_sparse_long_compressed_amd import synth
from oracle import cobs_oracle as O
from tests import gpu_util as U
from tests.test_gpu_parity import run_and_check
from tests.test_gpu_prefill import check_prefill
from tests.test_gpu_update import run_update, untouched_equal

pytestmark = pytest.mark.gpu

MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    yield


FP4 = dict(batch=2, max_len=1500, min_len=700, n_q_heads=8, n_kv_heads=2, head_dim=128, top_k=6,
           window=200, cmp_len=32, cmp_stride=16, so_kind="lowrank_fp4", rank=4, alpha=1.0, dtype="bf16",
           needles=2)


def unpack_records(rec: np.ndarray, rank: int, d: int):
    """Codes [.., rank, d] and exponents [.., rank, d/32] of stored records (the
    byte layout of the compressed storage: codes two per byte, low nibble first,
    entry 16u + 4g + c at nibble (g*d/16 + u)*4 + c; then the exponent bytes)."""
    lead = rec.shape[:-1]
    P = np.arange(d)
    g, kk = P // (d // 4), P % (d // 4)
    entry = 16 * (kk // 4) + 4 * g + kk % 4
    codes = np.zeros(lead + (rank, d), dtype=np.int64)
    for i in range(rank):
        cb = rec[..., i * (d // 2):(i + 1) * (d // 2)].astype(np.int64)
        nib = np.stack([cb & 0xF, cb >> 4], axis=-1).reshape(lead + (d,))
        codes[..., i, entry] = nib
    e0 = rank * (d // 2)
    exps = rec[..., e0:e0 + rank * (d // 32)].astype(np.int64).reshape(lead + (rank, d // 32)) - 127
    return codes, exps


def check_fp4(w, x, s, units=None, gap_min=1e-2):
    """Compressed summaries against the oracle's (see the module docstring); with a
    query subspace (w.subspace > 0, P = x["P"]) the vectors are those of P C P^T,
    stored with length vlen = s rounded up to 32."""
    p = O.params_of(w)
    d, r, G = w.head_dim, w.rank, w.group
    vlen = -(-w.subspace // 32) * 32 if w.subspace else d
    mu_dev = s["mu"]                       # blocks past a sequence's end are never written: sliced before any cast
    codes, exps = unpack_records(s["so"].cpu().numpy(), r, vlen)
    units = units or [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    strict = loose = exempt = total = mu_equal = mu_total = 0
    for (b, h) in units:
        print(f"[test] compressed summaries of unit ({b}, {h})", flush=True)
        L = int(x["lens"][b])
        keys = x["K"][b, h, :L].astype(np.float64)
        Ph = None if not w.subspace else x["P"][h].astype(np.float64)
        rmu, rso, n = O.summaries(keys, L, "lowrank_fp4", r, Ph)
        nb = len(n)
        mu_u = mu_dev[b, h, :nb].float().cpu().numpy().astype(np.float64)
        assert np.isfinite(mu_u).all(), (b, h)
        ulp = np.maximum(np.abs(rmu), 1e-38) * 2.0 ** -7
        assert (np.abs(mu_u - rmu) <= ulp * 1.0001).all(), (b, h)
        mu_equal += int((mu_u == rmu).sum())
        mu_total += rmu.size
        q = x["Q"][b, 0, h * G:(h + 1) * G].astype(np.float64) * p["scale"]
        if Ph is not None:
            q = q @ Ph.T                                          # coordinates in the subspace
        for blk in range(nb):
            kb = keys[blk * 64: blk * 64 + n[blk]]
            C = O.block_covariance(kb)
            if Ph is not None:
                C = Ph @ C @ Ph.T
                v_ref = O.subspace_second_order(kb, r, Ph)
            else:
                v_ref = O.lowrank_second_order(kb, r)
            lam = np.sort(np.linalg.eigvalsh(C))[::-1]
            v_ref = np.concatenate([v_ref, np.zeros((r, vlen - v_ref.shape[1]))], axis=1)
            if n[blk] > r + 1 and (lam[r - 1] - lam[r]) >= gap_min * lam[r - 1]:
                strict += 1
                for i in range(r):
                    c_ref, e_ref = O.quantize_mxfp4(v_ref[i])
                    c_got, e_got = codes[b, h, blk, i], exps[b, h, blk, i]
                    top2 = np.sort(np.abs(v_ref[i]))[-2:]
                    if top2[1] - top2[0] <= 1e-9 * top2[1] and (c_got != c_ref).sum() > vlen // 4:
                        c_got = np.where(c_got & 7, c_got ^ 8, c_got)         # sign convention tie
                    for gi in range(vlen // 32):
                        sl = slice(32 * gi, 32 * gi + 32)
                        amax = np.abs(v_ref[i, sl]).max()
                        total += 32
                        if amax == 0.0:
                            assert e_got[gi] == -127 and (c_got[sl] == 0).all(), (b, h, blk, i, gi)
                            continue
                        l2 = np.log2(amax)
                        if abs(l2 - np.round(l2)) < 1e-9:
                            exempt += 32
                            continue
                        assert e_got[gi] == e_ref[gi], (b, h, blk, i, gi)
                        y = np.abs(v_ref[i, sl]) / 2.0 ** e_ref[gi]
                        near = np.abs(y[:, None] - MIDS[None, :]).min(axis=1) < 1e-6
                        exempt += int(near.sum())
                        bad = (c_got[sl] != c_ref[sl]) & ~near
                        assert not bad.any(), (b, h, blk, i, gi, np.nonzero(bad))
            else:
                loose += 1
                got = O.dequantize_mxfp4(codes[b, h, blk].reshape(-1), exps[b, h, blk].reshape(-1))
                got = got.reshape(r, vlen)[:, :q.shape[1]]
                qg = np.einsum("hd,rd->hr", q, got)
                qr = np.einsum("hd,rd->hr", q, rso[blk])
                dq = (qg * qg).sum(1) - (qr * qr).sum(1)
                assert np.abs(dq).max() <= 1e-3 * max(1.0, float((qr * qr).sum(1).max())), (b, h, blk)
    assert strict > 0
    assert mu_equal >= 0.99 * mu_total
    assert exempt <= 1e-3 * total, (exempt, total)
    return strict, loose


@pytest.mark.parametrize("rank,d", [(4, 128), (1, 128), (8, 128), (3, 64)])
def test_summaries_fp4(rank, d):
    w = synth.Workload("fp4", **dict(FP4, rank=rank, head_dim=d, n_q_heads=2 * (4 if d == 128 else 8)))
    x = synth.make_inputs(w, 31, lens=np.array([1500, 700]))
    p = U.params_for(w)
    s = U.build(p, U.to_device(x))
    check_fp4(w, x, s)


@pytest.mark.parametrize("alpha", [0.0, 1.0])
def test_decode_fp4_small(alpha):
    w = synth.Workload("fp4", **FP4)
    x = synth.make_inputs(w, 32, lens=np.array([1500, 777]))
    run_and_check(w, x, alpha=alpha)


def test_decode_fp4_f32_d64():
    w = synth.Workload("fp4", **dict(FP4, head_dim=64, n_q_heads=16, dtype="f32", rank=2))
    x = synth.make_inputs(w, 33, lens=np.array([1300, 640]))
    run_and_check(w, x)


def test_prefill_fp4():
    L, T = 900, 64
    w = synth.Workload("pf4", **dict(FP4, batch=1, max_len=L, min_len=L, n_q_heads=16, n_q_tokens=T,
                                     q_pos0=L - T))
    x = synth.make_inputs(w, 34)
    check_prefill(w, x, tokens=list(range(T)))


def test_update_fp4():
    w = synth.Workload("upd4", **dict(FP4, max_len=1100, min_len=500))
    old_lens, new_lens = [1000, 511], [1090, 513]
    x, s, before = run_update(w, new_lens, old_lens, 90)
    check_fp4(w, x, s)
    untouched_equal(s, before, old_lens, w)


def test_full_size_long_decode_fp4(long_inputs, long_oracle_lowrank):
    """8 x 128k with the compressed storage: codes, exponents and means of 4 units,
    selections of 16 units over all 8 sequences and every kv head, outputs where the
    gap is unambiguous.  The oracle's compressed summaries are its fp64 rank-4
    summaries rounded (bf16 mean, MX FP4 vectors), as its summary builder does."""
    from tests.test_gpu_parity import check_long_units
    w = synth.WORKLOADS["decode_b8_L128k_rank4_fp4"]
    _, x = long_inputs
    x = dict(x, workload=w)
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    check_fp4(w, x, s, units=[(0, 0), (3, 1), (7, 5), (5, 3)])
    out, sel = U.decode(p, g, s)
    units = {}
    for key, ((mu, so, n), kc, vc) in long_oracle_lowrank.items():
        qmu = O.round_bf16(mu)
        qso = np.array([[O.quantize_dequantize_padded(v) for v in blk] for blk in so])
        units[key] = ((qmu, qso, n), kc, vc)
    check_long_units(w, x, out, sel, units, O.params_of(w))
