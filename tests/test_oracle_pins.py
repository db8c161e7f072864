"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test fixes one part of the method against a closed form, an exact
identity, a library routine that computes the same quantity by another
route (torch's float64 scaled-dot-product attention), brute force on tiny
inputs, or the worked picture of the COBS explainer (tests/golden/).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import cobs_oracle as O
from block_sparse_long_compressed_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa64(q, k, v, scale, mask=None):
    """torch float64 attention on the CPU: an independent softmax(qk)v route."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))[None, None]
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)[0, 0].numpy()


def gauss_hermite_log_mgf(mean, var, nodes=80):
    """ln E[exp(X)] for X ~ N(mean, var) by Gauss-Hermite quadrature."""
    x, wts = np.polynomial.hermite.hermgauss(nodes)
    return math.log(float((wts * np.exp(mean + math.sqrt(2.0 * var) * x)).sum() / math.sqrt(math.pi)))


# --------------------------------------------------------------------------
# Score: the cumulant expansion is exact for Gaussian keys (COBS sec. 2.2)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["diag", "lowrank"])
def test_score_matches_gaussian_log_mgf(kind):
    rng = np.random.default_rng(1)
    d, scale = 16, 1.0 / 4.0
    q = rng.standard_normal((3, d))
    mu = 0.3 * rng.standard_normal((1, d))
    if kind == "diag":
        so = rng.uniform(0.05, 1.5, size=(1, d))
        cov = np.diag(so[0])
    else:
        so = 0.6 * rng.standard_normal((1, 3, d))
        cov = so[0].T @ so[0]
    for n_b in (1, 7, 64):
        s = O.block_scores(q, mu, so, np.array([n_b]), alpha=1.0, scale=scale, so_kind=kind)
        for h in range(3):
            m = scale * q[h] @ mu[0]
            v = scale * scale * q[h] @ cov @ q[h]
            ref = math.log(n_b) + gauss_hermite_log_mgf(m, v)
            assert abs(s[h, 0] - ref) < 1e-10, (kind, n_b, h, s[h, 0], ref)


def test_alpha_weights_only_second_order_term():
    rng = np.random.default_rng(2)
    d, scale = 8, 0.5
    q = rng.standard_normal((2, d))
    mu = rng.standard_normal((4, d))
    so = rng.uniform(0.1, 1.0, (4, d))
    n = np.array([64, 64, 64, 10])
    s0 = O.block_scores(q, mu, so, n, 0.0, scale, "diag")
    s1 = O.block_scores(q, mu, so, n, 1.0, scale, "diag")
    s2 = O.block_scores(q, mu, so, n, 2.0, scale, "diag")
    # linear in alpha, and alpha = 0 drops every trace of the variance channel
    np.testing.assert_allclose(s2 - s1, s1 - s0, rtol=0, atol=1e-12)
    s0b = O.block_scores(q, mu, 100 * so, n, 0.0, scale, "diag")
    np.testing.assert_allclose(s0, s0b, rtol=0, atol=0)


# --------------------------------------------------------------------------
# Score: exact special cases on finite blocks
# --------------------------------------------------------------------------

def test_single_key_block_score_is_exact_log_mass():
    rng = np.random.default_rng(3)
    d, scale = 32, 1 / math.sqrt(32)
    for kind, r in (("diag", 0), ("lowrank", 4)):
        keys = rng.standard_normal((1, d))
        mu, so, n = O.summaries(keys, 1, kind, r)
        q = rng.standard_normal((1, d))
        s = O.block_scores(q, mu, so, n, 1.0, scale, kind)
        assert abs(s[0, 0] - math.log(O.attention_mass(q[0], keys, scale))) < 1e-12


@pytest.mark.parametrize("kind", ["diag", "lowrank"])
def test_two_point_block_ln_cosh(kind):
    """Keys centre +- delta (32 each): ln m_b = ln 64 + scale q.centre + ln cosh x,
    the second-order score has x^2/2 in place of ln cosh x, x = scale q.delta."""
    d, scale = 8, 0.25
    rng = np.random.default_rng(4)
    centre = rng.standard_normal(d)
    for a in (0.05, 0.5, 2.0):
        delta = np.zeros(d)
        delta[3] = a
        keys = np.vstack([np.tile(centre + delta, (32, 1)), np.tile(centre - delta, (32, 1))])
        mu, so, n = O.summaries(keys, 64, kind, 2)
        np.testing.assert_allclose(mu[0], centre, rtol=0, atol=1e-14)
        if kind == "diag":
            ref_var = np.zeros(d)
            ref_var[3] = a * a
            np.testing.assert_allclose(so[0], ref_var, rtol=0, atol=1e-14)
        else:
            np.testing.assert_allclose(so[0][0], np.abs(delta), rtol=0, atol=1e-12)
            np.testing.assert_allclose(so[0][1], 0.0, atol=1e-7)
        q = rng.standard_normal((1, d))
        x = scale * q[0] @ delta
        ln_m = math.log(O.attention_mass(q[0], keys, scale))
        assert abs(ln_m - (math.log(64) + scale * q[0] @ centre + math.log(math.cosh(x)))) < 1e-12
        s = O.block_scores(q, mu, so, n, 1.0, scale, kind)[0, 0]
        assert abs(s - (math.log(64) + scale * q[0] @ centre + 0.5 * x * x)) < 1e-12
        # truncation error of the second-order expansion: ln cosh x - x^2/2 = -x^4/12 + ...
        if abs(x) < 0.2:
            assert abs((ln_m - s) + x ** 4 / 12) < abs(x) ** 6


def test_equal_logits_make_lowrank_score_exact():
    """All q.k_r equal in the block -> kappa_2 q = 0 -> score = ln m_b exactly."""
    rng = np.random.default_rng(5)
    d, scale = 12, 0.3
    q = rng.standard_normal(d)
    basis = np.linalg.qr(np.column_stack([q, rng.standard_normal((d, d - 1))]))[0]
    perp = basis[:, 1:]                                   # orthogonal to q
    keys = rng.standard_normal(d) + rng.standard_normal((64, d - 1)) @ perp.T
    mu, so, n = O.summaries(keys, 64, "lowrank", 4)
    s = O.block_scores(q[None], mu, so, n, 1.0, scale, "lowrank")[0, 0]
    assert abs(s - math.log(O.attention_mass(q, keys, scale))) < 1e-10


def test_second_order_gap_shrinks_with_gaussian_block_size():
    """Gaussian keys: the estimate converges to ln m_b as n_b grows (trend check)."""
    rng = np.random.default_rng(6)
    d, scale = 16, 0.25
    q = rng.standard_normal(d)
    errs = []
    for n_b in (64, 4096, 262144):
        keys = 0.2 + 0.7 * rng.standard_normal((n_b, d))
        mu = keys.mean(0, keepdims=True)
        so = keys.var(0, keepdims=True)
        s = O.block_scores(q[None], mu, so, np.array([n_b]), 1.0, scale, "diag")[0, 0]
        errs.append(abs(s - math.log(O.attention_mass(q, keys, scale))))
    assert errs[2] < errs[0]


# --------------------------------------------------------------------------
# Summaries against constructed blocks with known moments
# --------------------------------------------------------------------------

def hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_lowrank_recovers_known_spectrum():
    """Keys = centre + sum_i H[:, i] s_i u_i with Hadamard columns (mean 0, mutually
    orthogonal) and orthonormal u_i: kappa_2 = sum_i s_i^2 u_i u_i^T exactly."""
    rng = np.random.default_rng(7)
    d = 32
    U = np.linalg.qr(rng.standard_normal((d, d)))[0]
    s = np.array([3.0, 2.0, 1.5, 1.0, 0.5, 0.25])
    H = hadamard(64)[:, 1:1 + len(s)]
    centre = rng.standard_normal(d)
    keys = centre + (H * s) @ U[:, :len(s)].T
    perm = rng.permutation(len(s))                      # insertion order must not matter
    keys2 = centre + (H[:, perm] * s[perm]) @ U[:, perm].T
    for kk in (keys, keys2):
        mu, so, n = O.summaries(kk, 64, "lowrank", 4)
        np.testing.assert_allclose(mu[0], centre, atol=1e-12)
        for i in range(4):
            v = so[0][i]
            ref = s[i] * U[:, i]                         # sqrt(eigenvalue) = s_i (1/n_b normalisation)
            assert min(np.abs(v - ref).max(), np.abs(v + ref).max()) < 1e-10
            assert v[np.argmax(np.abs(v))] > 0
    # diagonal channel of the same block is diag(kappa_2)
    mu, so, n = O.summaries(keys, 64, "diag", 0)
    np.testing.assert_allclose(so[0], ((U[:, :len(s)] * s) ** 2).sum(1), atol=1e-12)


def test_summaries_permutation_invariant_and_partial_block():
    rng = np.random.default_rng(8)
    d, L = 16, 64 * 3 + 5
    keys = rng.standard_normal((L, d))
    mu, so, n = O.summaries(keys, L, "diag", 0)
    assert list(n) == [64, 64, 64, 5]
    keys_p = keys.copy()
    keys_p[64:128] = keys[64:128][rng.permutation(64)]
    mu2, so2, _ = O.summaries(keys_p, L, "diag", 0)
    np.testing.assert_allclose(mu, mu2, atol=1e-14)
    np.testing.assert_allclose(so, so2, atol=1e-14)
    # trailing block uses only its 5 keys: constant keys there give zero variance
    keys_c = keys.copy()
    keys_c[192:] = 1.25
    mu3, so3, _ = O.summaries(keys_c, L, "diag", 0)
    np.testing.assert_allclose(mu3[3], 1.25, atol=1e-15)
    np.testing.assert_allclose(so3[3], 0.0, atol=1e-15)


def test_compressed_tokens_on_a_ramp():
    d = 3
    for L, nc in ((31, 0), (32, 1), (47, 1), (48, 2), (100, 5), (1024, 63)):
        x = np.repeat(np.arange(L, dtype=np.float64)[:, None], d, axis=1)
        kc = O.compressed_tokens(x, L, 32, 16)
        assert kc.shape == (nc, d)
        for j in range(nc):
            np.testing.assert_allclose(kc[j], 16 * j + 15.5, atol=1e-12)


# --------------------------------------------------------------------------
# Group aggregation and top-k
# --------------------------------------------------------------------------

def test_group_scores_sum_to_group_size_and_single_head_ranking():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((5, 40)) * 3
    shat = O.group_scores(s)
    assert abs(np.exp(shat).sum() - 5.0) < 1e-12           # each head's shares sum to 1
    one = O.group_scores(s[:1])
    assert abs(np.exp(one).sum() - 1.0) < 1e-12
    assert list(np.argsort(-one, kind="stable")) == list(np.argsort(-s[0], kind="stable"))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(10)
    for trial in range(200):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 10))
        shat = rng.integers(0, 4, size=n).astype(np.float64)    # many exact ties
        sel, gap = O.select_topk(shat, k)
        take = min(k, n)
        assert list(sel[take:]) == [-1] * (k - take)
        S = list(sel[:take])
        assert S == sorted(S) and len(set(S)) == take
        # brute force: the chosen set is the best of all size-`take` subsets under
        # the order (score desc, index asc) compared element-wise after sorting
        def key(sub):
            return sorted(((-shat[b], b) for b in sub))
        best = min(itertools.combinations(range(n), take), key=key)
        assert S == sorted(best)


def test_topk_gap_is_the_margin_between_chosen_and_rest():
    """The reported gap is the margin of the chosen set: the lowest chosen score minus
    the highest score left out (inf when nothing is left out), checked on random
    scores with many exact ties (gap 0 where the cut falls inside a tie)."""
    rng = np.random.default_rng(12)
    for trial in range(300):
        n = int(rng.integers(1, 12))
        k = int(rng.integers(1, 12))
        shat = rng.integers(0, 5, size=n).astype(np.float64) * 0.25
        sel, gap = O.select_topk(shat, k)
        chosen = [int(b) for b in sel if b >= 0]
        rest = [b for b in range(n) if b not in chosen]
        if not rest:
            assert gap == np.inf
        else:
            assert gap == min(shat[chosen]) - max(shat[rest])
            assert gap >= 0.0


def test_topk_gap_of_constant_blocks_is_the_logit_difference():
    """Blocks of 64 identical keys have zero covariance, so their score is exactly
    ln 64 + scale q.k_b; with one head the group score is that minus a common
    log-sum-exp, and the gap between the k-th and (k+1)-th block is the scaled
    difference of their logits: for keys c_b e_0 against q = e_0 at scale 1/8 and
    c = (0.5, 2.0, 1.25, 3.0, -1.0), k = 2 gives (2.0 - 1.25)/8 = 0.09375."""
    d = 64
    c = [0.5, 2.0, 1.25, 3.0, -1.0]
    keys = np.zeros((64 * len(c), d))
    for b, cb in enumerate(c):
        keys[64 * b: 64 * b + 64, 0] = cb
    vals = np.ones((64 * len(c), d))
    L = keys.shape[0]
    p = {"top_k": 2, "window": 0, "cmp_len": 0, "cmp_stride": 16, "so_kind": "diag", "rank": 0, "alpha": 1.0,
         "scale": 0.125}
    summ = O.summaries(keys, L, "diag")
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    out, sel, shat, gap = O.query_group(p, q, keys, vals, L, L - 1, summ, np.zeros((0, d)), np.zeros((0, d)), None)
    assert list(sel) == [1, 3]
    assert abs(gap - 0.09375) < 1e-14
    p["top_k"] = 5
    assert O.query_group(p, q, keys, vals, L, L - 1, summ, np.zeros((0, d)), np.zeros((0, d)), None)[3] == np.inf


def test_duplicate_blocks_tie_to_lower_index():
    rng = np.random.default_rng(11)
    d = 8
    blk = rng.standard_normal((64, d))
    keys = np.vstack([rng.standard_normal((64, d)) * 0.1, blk, blk, rng.standard_normal((64, d)) * 0.1])
    mu, so, n = O.summaries(keys, 256, "diag", 0)
    q = rng.standard_normal((2, d))
    s = O.block_scores(q, mu, so, n, 1.0, 0.35, "diag")
    shat = O.group_scores(s)
    assert shat[1] == shat[2]
    order = sorted(range(4), key=lambda b: (-shat[b], b))
    if order[0] in (1, 2):
        sel, _ = O.select_topk(shat, 1)
        assert sel[0] == 1


def test_bundle_example_from_the_explainer():
    g = json.load(open(os.path.join(GOLDEN, "bundle_example.json")))
    d, scale = g["d"], g["scale"]
    q = np.array(g["query"])[None]
    c = np.array(g["centre"])
    keys = []
    for name in g["block_order"]:
        dl = np.array(g["delta"][name])
        keys += [c + dl] * 32 + [c - dl] * 32
    keys = np.array(keys)
    mu, so, n = O.summaries(keys, 128, "diag", 0)
    s0 = O.block_scores(q, mu, so, n, 0.0, scale, "diag")
    s1 = O.block_scores(q, mu, so, n, 1.0, scale, "diag")
    assert s0[0, 0] == s0[0, 1]
    assert list(O.select_topk(O.group_scores(s0), g["top_k"])[0]) == g["expect"]["first_order_alpha0"]["selected"]
    assert list(O.select_topk(O.group_scores(s1), g["top_k"])[0]) == g["expect"]["second_order_alpha1"]["selected"]
    p = {"scale": scale, "top_k": g["top_k"]}
    assert list(O.oracle_selection_mass(p, q, keys, 128, 127)) == g["expect"]["exact_mass_selected"]


# --------------------------------------------------------------------------
# Branch attention, combine, end-to-end reductions to dense attention
# --------------------------------------------------------------------------

def tiny_inputs(L=600, d=16, G=3, kind="diag", seed=12):
    w = synth.Workload("t", 1, L, L, G, 1, d, 4, 0, 0, 16, kind, 2, 1.0, "f32", 1, gates=False)
    return w, synth.make_inputs(w, seed)


def test_topk_all_blocks_equals_dense_attention():
    for kind in ("diag", "lowrank"):
        w, x = tiny_inputs(kind=kind)
        L = int(x["lens"][0])
        p = O.params_of(w)
        p["top_k"] = O.num_blocks(L)
        out = O.run(x, p)[(0, 0, 0)][0]
        K = x["K"][0, 0, :L].astype(np.float64)
        V = x["V"][0, 0, :L].astype(np.float64)
        for h in range(w.group):
            ref = sdpa64(x["Q"][0, 0, h][None], K, V, p["scale"])[0]
            np.testing.assert_allclose(out[h], ref, rtol=0, atol=1e-12)


def test_block_mass_fractions_match_attention_with_block_indicator_values():
    rng = np.random.default_rng(13)
    d, L, scale = 8, 64 * 4 + 9, 0.4
    keys = rng.standard_normal((L, d))
    q = rng.standard_normal(d)
    n = O.block_sizes(L)
    ind = np.zeros((L, len(n)))
    for b in range(len(n)):
        ind[b * 64: b * 64 + n[b], b] = 1.0
    frac = sdpa64(q[None], keys, ind, scale)[0]
    m = np.array([O.attention_mass(q, keys[b * 64: b * 64 + n[b]], scale) for b in range(len(n))])
    np.testing.assert_allclose(m / m.sum(), frac, rtol=1e-12, atol=0)


def prefill_inputs(L=700, T=40, d=16, G=2, W=100, seed=14):
    w = synth.Workload("p", 1, L, L, G, 1, d, 3, W, 32, 16, "diag", 0, 1.0, "f32", 2,
                       n_q_tokens=T, q_pos0=L - T)
    return w, synth.make_inputs(w, seed)


def test_window_branch_is_causal_banded_attention():
    w, x = prefill_inputs()
    p = O.params_of(w)
    x["gates"][:] = np.array([0.0, 0.0, 1.0], dtype=np.float32)
    L = int(x["lens"][0])
    K = x["K"][0, 0, :L].astype(np.float64)
    V = x["V"][0, 0, :L].astype(np.float64)
    res = O.run(x, p, tokens=[0, 17, w.n_q_tokens - 1])
    for i in (0, 17, w.n_q_tokens - 1):
        t = w.q_pos0 + i
        mask = np.zeros((1, L), dtype=bool)
        mask[0, max(0, t - w.window + 1): t + 1] = True
        for h in range(w.group):
            ref = sdpa64(x["Q"][0, i, h][None], K, V, p["scale"], mask)[0]
            np.testing.assert_allclose(res[(0, 0, i)][0][h], ref, atol=1e-12)


def test_selected_branch_with_all_candidates_is_causal_block_attention():
    w, x = prefill_inputs()
    p = O.params_of(w)
    p["top_k"] = O.num_blocks(w.max_len)
    x["gates"][:] = np.array([0.0, 1.0, 0.0], dtype=np.float32)
    L = int(x["lens"][0])
    K = x["K"][0, 0, :L].astype(np.float64)
    V = x["V"][0, 0, :L].astype(np.float64)
    res = O.run(x, p, tokens=[0, 3, 39])
    for i in (0, 3, 39):
        t = w.q_pos0 + i
        # only blocks whose every key is at or before t; at t = L-1 that
        # includes the trailing partial block
        visible = L if t == L - 1 else ((t + 1) // 64) * 64
        mask = np.zeros((1, L), dtype=bool)
        mask[0, :visible] = True
        for h in range(w.group):
            ref = sdpa64(x["Q"][0, i, h][None], K, V, p["scale"], mask)[0]
            np.testing.assert_allclose(res[(0, 0, i)][0][h], ref, atol=1e-12)


def test_compressed_branch_attends_over_visible_pooled_tokens():
    w, x = prefill_inputs()
    p = O.params_of(w)
    x["gates"][:] = np.array([1.0, 0.0, 0.0], dtype=np.float32)
    L = int(x["lens"][0])
    K = x["K"][0, 0, :L].astype(np.float64)
    V = x["V"][0, 0, :L].astype(np.float64)
    res = O.run(x, p, tokens=[0, 20])
    for i in (0, 20):
        t = w.q_pos0 + i
        nvis = (t - 31) // 16 + 1
        kc = np.array([K[16 * j: 16 * j + 32].sum(0) / 32 for j in range(nvis)])
        vc = np.array([V[16 * j: 16 * j + 32].sum(0) / 32 for j in range(nvis)])
        for h in range(w.group):
            ref = sdpa64(x["Q"][0, i, h][None], kc, vc, p["scale"])[0]
            np.testing.assert_allclose(res[(0, 0, i)][0][h], ref, atol=1e-12)


def test_gated_combine_is_linear_in_the_gates():
    w, x = prefill_inputs(T=3)
    p = O.params_of(w)
    outs = []
    for g in np.eye(3):
        x["gates"][:] = g.astype(np.float32)
        outs.append(O.run(x, p)[(0, 0, 2)][0])
    gm = np.array([0.3, 0.5, 0.9], dtype=np.float32)
    x["gates"][:] = gm
    mixed = O.run(x, p)[(0, 0, 2)][0]
    np.testing.assert_allclose(mixed, sum(float(gm[i]) * outs[i] for i in range(3)), atol=1e-12)
    # each branch output is a convex combination of its values
    V = x["V"][0, 0].astype(np.float64)
    for o in outs:
        assert (o <= V.max(0) + 1e-12).all() and (o >= V.min(0) - 1e-12).all()


def test_prefill_at_last_position_equals_decode():
    L = 640
    base = dict(batch=1, max_len=L, min_len=L, n_q_heads=4, n_kv_heads=2, head_dim=16, top_k=3,
                window=100, cmp_len=32, cmp_stride=16, so_kind="diag", rank=0, alpha=1.0,
                dtype="f32", needles=1)
    wd = synth.Workload("d", **base)
    wp = synth.Workload("p", **base, n_q_tokens=1, q_pos0=L - 1)
    xd = synth.make_inputs(wd, 15)
    xp = dict(xd, workload=wp)
    rd = O.run(xd, O.params_of(wd))
    rp = O.run(xp, O.params_of(wp))
    for g in range(2):
        np.testing.assert_array_equal(rd[(0, g, 0)][1], rp[(0, g, 0)][1])
        np.testing.assert_allclose(rd[(0, g, 0)][0], rp[(0, g, 0)][0], atol=0)


def test_fewer_candidates_than_k_pads_with_minus_one():
    w, x = prefill_inputs(L=200, T=150, W=16)
    p = O.params_of(w)
    r = O.run(x, p, tokens=[0])[(0, 0, 0)]               # t = 50: no complete block yet
    assert list(r[1]) == [-1, -1, -1]
    r = O.run(x, p, tokens=[100])[(0, 0, 100)]           # t = 150: blocks 0, 1 complete
    assert list(r[1]) == [0, 1, -1]


def test_second_order_recall_against_exact_mass_beats_first_order():
    """Directional claim of the COBS explainer (sec. 2.2, 4.1): adding the
    covariance term brings the selection closer to ranking by exact mass (OSA).
    Summed over seeds on the tiny mixture workload, recall at alpha = 1 must
    exceed recall at alpha = 0 (the mean-pool selector)."""
    w = synth.WORKLOADS["tiny_f32_L1k"]
    rec1 = rec0 = 0
    for seed in range(8):
        x = synth.make_inputs(w, seed)
        osa = set(O.oracle_selection_mass(O.params_of(w), x["Q"][0, 0].astype(np.float64),
                                          x["K"][0, 0].astype(np.float64), 1024, 1023))
        rec1 += len(osa & set(O.run(x, O.params_of(w))[(0, 0, 0)][1]))
        rec0 += len(osa & set(O.run(x, O.params_of(w, alpha=0.0))[(0, 0, 0)][1]))
    assert rec1 > rec0, (rec1, rec0)


# ---------------------------------------------------------------------------
# Compressed summary storage ([COBS] 2.3: BF16 mean, FP4 eigenvectors) with the
# OCP microscaling (MX) FP4 rule: per 32 entries X = 2^(floor(log2 amax) - 2),
# entries rounded to E2M1 {0, .5, 1, 1.5, 2, 3, 4, 6} * X, ties to the even code.
# ---------------------------------------------------------------------------

def test_e2m1_grid_ties_and_saturation():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for code, v in enumerate(grid):
        assert O.quantize_e2m1(v) == code
        if code:
            assert O.quantize_e2m1(-v) == 8 | code
    # midpoints go to the code with a zero mantissa bit (the even code)
    for mid, code in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]:
        assert O.quantize_e2m1(mid) == code, mid
    # just off a midpoint, the nearer value wins
    assert O.quantize_e2m1(1.2500001) == 3 and O.quantize_e2m1(4.9999) == 6
    # saturation and signed zero
    assert O.quantize_e2m1(7.99) == 7 and O.quantize_e2m1(-100.0) == 15
    assert O.quantize_e2m1(-0.1) == 0


def test_mx_group_scale_hand_example():
    g = np.zeros(32)
    g[0], g[1], g[2], g[3] = 3.0, 0.3, -1.1, 0.12
    codes, exps = O.quantize_mxfp4(g)
    assert exps.tolist() == [-1]                       # floor(log2 3) - 2 = -1: X = 1/2
    # 3 -> 6X (code 7); .3 -> .6X -> .5X (code 1); -1.1 -> -2.2X -> -2X (code 12); .12 -> .24X -> 0
    assert codes[:4].tolist() == [7, 1, 12, 0]
    assert O.dequantize_mxfp4(codes, exps)[:4].tolist() == [3.0, 0.25, -1.0, 0.0]
    z, ez = O.quantize_mxfp4(np.zeros(32))
    assert not z.any() and not O.dequantize_mxfp4(z, ez).any()


def test_mxfp4_error_bound():
    """Half the local grid step: at most X below 6X, under 2X in the saturated top."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        v = rng.standard_normal(64) * 10.0 ** rng.uniform(-3, 2)
        codes, exps = O.quantize_mxfp4(v)
        err = np.abs(O.dequantize_mxfp4(codes, exps) - v)
        X = np.repeat(2.0 ** exps, 32)
        assert (err <= np.where(np.abs(v) <= 6 * X, 1.0, 2.0) * X + 1e-300).all()
        amax = np.abs(v).reshape(-1, 32).max(axis=1)
        assert ((amax >= 4 * 2.0 ** exps) & (amax < 8 * 2.0 ** exps)).all()


def test_round_bf16():
    assert O.round_bf16(np.array([1.0, -2.0, 0.0, 2.0 ** -130])).tolist() == [1.0, -2.0, 0.0, 2.0 ** -130]
    # halfway between 1 and 1 + 2^-7 goes to the even mantissa (1), between 1 + 2^-7 and 1 + 2^-6 up
    assert O.round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])).tolist() == [1.0, 1 + 2.0 ** -6]
    rng = np.random.default_rng(4)
    x = rng.standard_normal(1000) * 10.0 ** rng.uniform(-5, 5, 1000)
    r = O.round_bf16(x)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(x))) - 7)
    assert (np.abs(r - x) <= ulp / 2).all()


def test_fp4_summaries_are_the_rounded_lowrank_ones():
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((150, 64)) * 0.4 + 0.1
    mu, so, n = O.summaries(keys, 150, "lowrank", 2)
    mu4, so4, n4 = O.summaries(keys, 150, "lowrank_fp4", 2)
    assert (n == n4).all()
    np.testing.assert_array_equal(mu4, O.round_bf16(mu))
    for b in range(len(n)):
        for i in range(2):
            np.testing.assert_array_equal(so4[b, i], O.dequantize_mxfp4(*O.quantize_mxfp4(so[b, i])))
    # scores from the stored form stay close to the fp64 ones
    q = rng.standard_normal((4, 64))
    s32 = O.block_scores(q, mu, so, n, 1.0, 0.125, "lowrank")
    s4 = O.block_scores(q, mu4, so4, n4, 1.0, 0.125, "lowrank_fp4")
    assert np.abs(s4 - s32).max() < 0.05 * np.abs(s32).max()


# --------------------------------------------------------------------------
# Query-subspace projection (COBS sec. 2.3, "Subraum-Projektion")
# --------------------------------------------------------------------------

def test_query_subspace_of_a_known_second_moment():
    """Queries = rows of H diag(sigma) U^T with a Hadamard H (H^T H = N I): the
    sample second moment is U diag(sigma^2) U^T exactly, so P is the columns of U
    with the s largest sigma, largest first, each signed by its largest entry."""
    rng = np.random.default_rng(21)
    d, N, s = 16, 64, 5
    U = np.linalg.qr(rng.standard_normal((d, d)))[0]
    sigma = np.array([0.3, 2.5, 0.1, 1.7, 0.9, 3.1, 0.05, 1.2, 0.4, 0.6, 0.2, 0.8, 0.15, 1.0, 0.7, 0.5])
    H = hadamard(N)[:, :d]
    Q = (H * sigma) @ U.T
    P = O.query_subspace(Q, s)
    assert P.shape == (s, d)
    for i, j in enumerate(np.argsort(-sigma)[:s]):
        u = U[:, j] * np.sign(U[np.argmax(np.abs(U[:, j])), j])
        np.testing.assert_allclose(P[i], u, atol=1e-12)
    np.testing.assert_allclose(P @ P.T, np.eye(s), atol=1e-12)


def test_full_orthogonal_subspace_leaves_the_scores_unchanged():
    """s = d with an orthogonal P: (Pq)^T (P C P^T)_r (Pq) = q^T C_r q, because the top-r
    eigenvectors of P C P^T are P times those of C; the vectors are P v_i up to sign."""
    rng = np.random.default_rng(22)
    d, L, r = 16, 150, 3
    keys = rng.standard_normal((L, d)) * rng.uniform(0.2, 2.0, d)
    q = rng.standard_normal((4, d))
    P = np.linalg.qr(rng.standard_normal((d, d)))[0].T
    mu0, so0, n0 = O.summaries(keys, L, "lowrank", r)
    mu1, so1, n1 = O.summaries(keys, L, "lowrank", r, P)
    s0 = O.block_scores(q, mu0, so0, n0, 1.0, 0.25, "lowrank")
    s1 = O.block_scores(q, mu1, so1, n1, 1.0, 0.25, "lowrank", P)
    np.testing.assert_allclose(s1, s0, atol=1e-11)
    for b in range(len(n0)):
        for i in range(r):
            pv = P @ so0[b, i]
            assert min(np.abs(so1[b, i] - pv).max(), np.abs(so1[b, i] + pv).max()) < 1e-10


def test_subspace_query_with_full_rank_sees_the_whole_covariance():
    """q in span(P) (q = P^T a) and r = s: the quadratic term is exactly q^T kappa_2 q,
    the full second-order term, whatever the covariance outside the subspace."""
    rng = np.random.default_rng(23)
    d, s = 32, 6
    P = np.linalg.qr(rng.standard_normal((d, d)))[0][:, :s].T
    keys = rng.standard_normal((64, d)) * rng.uniform(0.1, 2.0, d) + rng.standard_normal(d)
    a = rng.standard_normal((3, s))
    q = a @ P
    mu, so, n = O.summaries(keys, 64, "lowrank", s, P)
    got = O.block_scores(q, mu, so, n, 1.0, 1.0, "lowrank", P)[:, 0]
    C = O.block_covariance(keys)
    ref = np.log(64) + q @ keys.mean(0) + 0.5 * np.einsum("hd,de,he->h", q, C, q)
    np.testing.assert_allclose(got, ref, atol=1e-10)


def test_covariance_orthogonal_to_the_subspace_gives_the_first_order_score():
    """Keys varying only in directions orthogonal to P: the projected covariance is 0,
    so every block scores like the alpha = 0 (mean-pool) selector."""
    rng = np.random.default_rng(24)
    d, s = 16, 4
    B = np.linalg.qr(rng.standard_normal((d, d)))[0]
    P = B[:, :s].T
    keys = rng.standard_normal(d) + rng.standard_normal((130, d - s)) @ B[:, s:].T
    q = rng.standard_normal((2, d))
    mu, so, n = O.summaries(keys, 130, "lowrank", 3, P)
    assert np.abs(so).max() < 1e-7                       # sqrt of rounding-level eigenvalues
    got = O.block_scores(q, mu, so, n, 1.0, 0.5, "lowrank", P)
    ref = O.block_scores(q, mu, so, n, 0.0, 0.5, "lowrank", P)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_subspace_fp4_pads_to_the_mx_group():
    """s = 20: each vector is quantized as 32 entries (12 zeros appended), so its
    stored value is the MX quantization of the padded vector, cut to 20 entries."""
    rng = np.random.default_rng(25)
    d, s = 32, 20
    P = np.linalg.qr(rng.standard_normal((d, d)))[0][:, :s].T
    keys = rng.standard_normal((64, d)) * 0.7
    _, so32, _ = O.summaries(keys, 64, "lowrank", 2, P)
    _, so4, _ = O.summaries(keys, 64, "lowrank_fp4", 2, P)
    for i in range(2):
        v = so32[0, i]
        e = int(np.floor(np.log2(np.abs(v).max()))) - 2
        ref = np.array([O.E2M1[O.quantize_e2m1(y / 2.0 ** e) & 7] * (1 if y >= 0 else -1) for y in v]) * 2.0 ** e
        np.testing.assert_allclose(so4[0, i], ref, atol=0)
