"""fp64 CPU oracle for COBS block-sparse attention (decode and chunked prefill).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module.  It shares no code with the HIP path
(no headers, helpers, tables or constants) and imports nothing from it; the two
meet only through the seeded input generator, which holds none of the method.

Plain and slow on purpose: numpy in float64, one (sequence, kv-head group,
query position) at a time, library primitives (matmul, eigh, sort) used as
single steps with no blocking or fusion.

Sources, cited by page title and section:
  [COBS]  "COBS: Cumulant Order Block Sparse Attention" (gist.science explainer,
          part "Technisches Resuemee"): sec. 2.1 selection criterion (attention
          mass m_b of a block), sec. 2.2 cumulant expansion of ln m_b with
          kappa_1 = block mean of the keys and kappa_2 = within-block key
          covariance, sec. 2.3 second-order score and covariance compression
          (top-r eigenvectors scaled by their eigenvalues), NoPE.
  [SKILL] "cumulant-order-block-sparse-attention" skill card: "Method" (keep the
          top-k blocks by the cumulant-aware mass estimate), "Implementation
          steps" (score = first-order term + alpha * cumulant term).
  [NSA]   GitHub issue "four dimensions regarding importance and connection
          strength" (Janus #181): the three branches (compression path,
          selection path, sliding window) and their gates g_cmp, g_slc.

Readings where the pages are silent or disagree (each one is listed with its
reason in the design notes of the repository):
  * temperature: logits are scale * q.k with scale = 1/sqrt(d) unless given,
    so the linear term carries scale and the quadratic term scale^2;
  * the quadratic term is weighted alpha * 1/2 (alpha = 1 is the truncated
    expansion of [COBS] 2.2, alpha = 0 the first-order mean-pool selector);
  * "ln L" in the expansion is ln n_b, the number of keys in block b;
  * kappa_2 uses 1/n_b (population covariance of the block's keys);
  * the compressed second-order channel is either the diagonal of kappa_2
    ('diag') or its top-r eigenvectors scaled by sqrt(eigenvalue) ('lowrank');
  * the compressed storage of [COBS] 2.3 (bf16 mean, FP4 eigenvectors;
    'lowrank_fp4') rounds the mean to the nearest bf16 (ties to even) and each
    scaled eigenvector to FP4 E2M1 with one power-of-two scale per 32
    consecutive entries, the scale and rounding of the OCP microscaling (MX)
    format: X = 2^(floor(log2 max|v|) - 2), entries round to the nearest of
    {0, .5, 1, 1.5, 2, 3, 4, 6} * X (ties to the even code), saturating at 6X;
  * the query-subspace projection of [COBS] 2.3 ("Subraum-Projektion") takes
    P [s][d] = the top-s eigenvectors of the queries' uncentred second moment
    E[q q^T] (rows signed so the largest-magnitude entry is positive), projects
    each block covariance into that subspace, C' = P kappa_2 P^T (s x s), and
    keeps the top-r scaled eigenvectors of C' (length s); the quadratic term is
    then sum_i ((P q) . v_i)^2, the linear term stays q . mu in full dimension;
    with the compressed storage the length-s vectors are padded with zeros to a
    multiple of 32 before the MX quantization;
  * a GQA group ranks blocks by the sum over its heads of each head's
    estimated share of attention mass (softmax of the scores over candidates);
  * ties go to the lower block index; fewer candidates than k -> pad with -1;
  * a block is a candidate for a query at position t iff all its keys are <= t
    (decode at t = L-1: every block, the trailing partial one included);
  * the compressed branch attends over means of 32 consecutive keys taken every
    16 positions, token j covering [16j, 16j+32), visible iff 16j+31 <= t;
  * the sliding window covers positions [max(0, t-W+1), t];
  * each branch is an exact softmax over its own key set; an empty set gives 0;
    output = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win (gates given as inputs).
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


# ----------------------------------------------------------------------------
# Blocks and per-block summaries  ([COBS] 2.1-2.3)
# ----------------------------------------------------------------------------

def num_blocks(L: int, block: int = BLOCK) -> int:
    """Blocks of `block` contiguous keys covering positions [0, L)."""
    return -(-L // block)


def block_sizes(L: int, block: int = BLOCK) -> np.ndarray:
    """n_b for every block; the trailing block may be partial."""
    nb = num_blocks(L, block)
    return np.array([min(block, L - b * block) for b in range(nb)], dtype=np.int64)


def block_mean(keys: np.ndarray) -> np.ndarray:
    """kappa_1 of a block: the mean of its keys ([COBS] 2.2)."""
    return keys.mean(axis=0)


def block_covariance(keys: np.ndarray) -> np.ndarray:
    """kappa_2 of a block: the covariance of its keys, normalised by n_b."""
    x = keys - block_mean(keys)
    return x.T @ x / keys.shape[0]


def diag_second_order(keys: np.ndarray) -> np.ndarray:
    """Diagonal compression of kappa_2: the per-coordinate variance."""
    return np.diag(block_covariance(keys)).copy()


def top_scaled_eigenvectors(cov: np.ndarray, rank: int) -> np.ndarray:
    """The `rank` largest eigenpairs (lambda_i, u_i) of a symmetric PSD matrix as
    v_i = sqrt(lambda_i) * u_i ([COBS] 2.3, "Low-Rank-Faktorisierung"), so that
    sum_i v_i v_i^T is its best rank-r approximation.  Eigenvalues <= 0 give
    v_i = 0.  Each v_i is signed so its largest-magnitude entry is positive (sign
    is irrelevant to the score; fixed only for reporting).  Returns [rank][n]."""
    lam, U = np.linalg.eigh(cov)            # ascending eigenvalues
    order = np.argsort(-lam, kind="stable")[:rank]
    out = np.zeros((rank, cov.shape[0]))
    for i, j in enumerate(order):
        if lam[j] > 0.0:
            v = np.sqrt(lam[j]) * U[:, j]
            if v[np.argmax(np.abs(v))] < 0:
                v = -v
            out[i] = v
    return out


def lowrank_second_order(keys: np.ndarray, rank: int) -> np.ndarray:
    """Low-rank compression of kappa_2: its top-r scaled eigenvectors, [rank][d]."""
    return top_scaled_eigenvectors(block_covariance(keys), rank)


def query_subspace(queries: np.ndarray, s: int) -> np.ndarray:
    """Query subspace of [COBS] 2.3 ("Subraum-Projektion"): the top-s eigenvectors
    of the queries' second moment M = (1/N) sum q q^T (uncentred), as the rows of
    P [s][d], each signed so its largest-magnitude entry is positive."""
    M = queries.T @ queries / queries.shape[0]
    lam, U = np.linalg.eigh(M)
    order = np.argsort(-lam, kind="stable")[:s]
    P = U[:, order].T.copy()
    for i in range(s):
        if P[i, np.argmax(np.abs(P[i]))] < 0:
            P[i] = -P[i]
    return P


def subspace_second_order(keys: np.ndarray, rank: int, P: np.ndarray) -> np.ndarray:
    """kappa_2 projected into the query subspace, C' = P kappa_2 P^T, compressed to
    its top-r scaled eigenvectors: [rank][s]."""
    return top_scaled_eigenvectors(P @ block_covariance(keys) @ P.T, rank)


# FP4 E2M1 magnitudes by code (sign in the fourth bit): 0, .5, 1, 1.5, 2, 3, 4, 6
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_GROUP = 32


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 of each value (ties to an even mantissa), as float64: the
    storage rounding of the compressed mean ([COBS] 2.3, BF16 mean)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for i, v in np.ndenumerate(x):
        if v == 0.0:
            out[i] = 0.0
            continue
        e = int(np.floor(np.log2(abs(v))))
        ulp = 2.0 ** (e - 7)                           # 8 significant bits
        q = v / ulp
        f = np.floor(q)
        r = q - f
        if r > 0.5 or (r == 0.5 and int(f) % 2 == 1):
            f += 1
        out[i] = f * ulp
    return out


def quantize_e2m1(y: float) -> int:
    """FP4 E2M1 code (0..15) of y (already divided by the group scale): nearest
    representable magnitude, ties to the even code, saturating at 6."""
    a = abs(y)
    sign = 8 if y < 0 else 0
    best = 0
    for c in range(8):
        d, db = abs(a - E2M1[c]), abs(a - E2M1[best])
        if d < db or (d == db and c % 2 == 0):
            best = c
    if a >= E2M1[7]:
        best = 7
    return sign | best if best else 0


def mx_scale_exponent(group: np.ndarray) -> int:
    """Shared power-of-two exponent of an MX group: floor(log2(max|v|)) - 2, so
    the largest entry lands in [4, 8) before rounding (E2M1's top binade)."""
    amax = float(np.max(np.abs(group)))
    if amax == 0.0:
        return -127
    return int(np.floor(np.log2(amax))) - 2


def quantize_mxfp4(v: np.ndarray):
    """Codes and group exponents of a vector (length a multiple of 32)."""
    codes = np.zeros(v.shape[0], dtype=np.int64)
    exps = np.zeros(v.shape[0] // MX_GROUP, dtype=np.int64)
    for gi in range(exps.shape[0]):
        grp = v[gi * MX_GROUP:(gi + 1) * MX_GROUP]
        e = mx_scale_exponent(grp)
        exps[gi] = e
        for j, y in enumerate(grp):
            codes[gi * MX_GROUP + j] = quantize_e2m1(y / 2.0 ** e)
    return codes, exps


def dequantize_mxfp4(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    mag = E2M1[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    return mag * np.repeat(2.0 ** exps.astype(np.float64), MX_GROUP)


def summaries(keys: np.ndarray, L: int, so_kind: str, rank: int = 0, P: np.ndarray | None = None):
    """Per-block summaries of one (sequence, kv-head): (mu [NB][d], so, n [NB]).

    so is [NB][d] for 'diag', [NB][rank][d] for 'lowrank' and for 'lowrank_fp4'
    (whose mean and vectors are the stored, rounded values).  With a query
    subspace P [s][d] (low-rank kinds only) the vectors have length s."""
    n = block_sizes(L)
    mu, so = [], []
    for b, nb in enumerate(n):
        kb = keys[b * BLOCK: b * BLOCK + nb]
        m = block_mean(kb)
        if so_kind == "diag":
            assert P is None, "the query subspace applies to the low-rank kinds"
            so.append(diag_second_order(kb))
        elif so_kind in ("lowrank", "lowrank_fp4"):
            v = lowrank_second_order(kb, rank) if P is None else subspace_second_order(kb, rank, P)
            if so_kind == "lowrank_fp4":
                m = round_bf16(m)
                v = np.array([quantize_dequantize_padded(x) for x in v])
            so.append(v)
        else:
            raise ValueError(so_kind)
        mu.append(m)
    return np.array(mu), np.array(so), n


def quantize_dequantize_padded(v: np.ndarray) -> np.ndarray:
    """The stored value of a vector in the compressed storage: zero-padded to a
    multiple of the MX group, quantized, dequantized, cut back to its length."""
    pad = -len(v) % MX_GROUP
    x = np.concatenate([v, np.zeros(pad)])
    return dequantize_mxfp4(*quantize_mxfp4(x))[:len(v)]


def compressed_tokens(x: np.ndarray, L: int, cmp_len: int = 32, cmp_stride: int = 16) -> np.ndarray:
    """Mean-pooled tokens for the compression branch ([NSA] compression path,
    mean pooling as in [COBS] 1): token j is the mean of positions
    [j*stride, j*stride + cmp_len), for every j whose span lies inside [0, L)."""
    if L < cmp_len:
        return np.zeros((0, x.shape[1]))
    nc = (L - cmp_len) // cmp_stride + 1
    return np.array([x[j * cmp_stride: j * cmp_stride + cmp_len].mean(axis=0) for j in range(nc)])


# ----------------------------------------------------------------------------
# Scoring, group aggregation, top-k  ([COBS] 2.1-2.3, [SKILL] Method)
# ----------------------------------------------------------------------------

def attention_mass(q: np.ndarray, keys: np.ndarray, scale: float) -> float:
    """Exact attention mass of a block, m_b = sum_r exp(scale * q.k_r) ([COBS] 2.1)."""
    return float(np.exp(scale * (keys @ q)).sum())


def block_scores(q: np.ndarray, mu: np.ndarray, so: np.ndarray, n: np.ndarray,
                 alpha: float, scale: float, so_kind: str, P: np.ndarray | None = None) -> np.ndarray:
    """Cumulant estimate of ln m_b for every query head and block ([COBS] 2.2, 2.3):

        s[h, b] = ln n_b + scale * q_h . mu_b + alpha * 1/2 * scale^2 * q_h^T S_b q_h

    with S_b = diag(so_b) ('diag') or sum_i so_b[i] so_b[i]^T ('lowrank'); with a
    query subspace P the quadratic term is (P q_h)^T S_b (P q_h), S_b built from
    the length-s vectors.  q is [H][d]; returns [H][NB]."""
    lin = scale * (q @ mu.T)
    if so_kind == "lowrank_fp4":
        so_kind = "lowrank"                                    # the stored vectors, dequantized
    if so_kind == "diag":
        quad = (q * q) @ so.T                                  # sum_j q_j^2 var_j
    else:
        qp = q if P is None else q @ P.T                       # coordinates of q in the subspace
        proj = np.einsum("hd,brd->hbr", qp, so)                # q . v_{b,i}
        quad = (proj * proj).sum(axis=2)
    return np.log(n.astype(np.float64))[None, :] + lin + alpha * 0.5 * scale * scale * quad


def logsumexp(x: np.ndarray, axis: int) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=axis, keepdims=True))).squeeze(axis)


def group_scores(s: np.ndarray) -> np.ndarray:
    """Rank score of each candidate block for a GQA group: the log of the sum
    over heads of the head's estimated share of attention mass in the block,
    share_h(b) = exp(s[h,b]) / sum_b' exp(s[h,b']).  s is [G][NBc]."""
    lse = logsumexp(s, axis=1)
    return logsumexp(s - lse[:, None], axis=0)


def select_topk(shat: np.ndarray, k: int):
    """Top-k blocks by group score, ties to the lower index ([SKILL] Method).

    Returns (selected indices in ascending order, padded with -1 to length k,
    gap = shat of the k-th pick minus shat of the (k+1)-th, inf if none)."""
    nc = shat.shape[0]
    order = sorted(range(nc), key=lambda b: (-shat[b], b))
    take = min(k, nc)
    chosen = sorted(order[:take])
    sel = np.full(k, -1, dtype=np.int64)
    sel[:take] = chosen
    gap = float(shat[order[take - 1]] - shat[order[take]]) if take < nc and take > 0 else np.inf
    return sel, gap


# ----------------------------------------------------------------------------
# Branch attention and gated combine  ([NSA] three paths and gates)
# ----------------------------------------------------------------------------

def softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """Exact softmax attention of one query head over one key set; 0 if empty."""
    if keys.shape[0] == 0:
        return np.zeros(vals.shape[1])
    logits = scale * (keys @ q)
    w = np.exp(logits - logits.max())
    w /= w.sum()
    return w @ vals


def dense_attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """Full softmax attention over all keys (what block sparsity avoids)."""
    return softmax_attend(q, keys, vals, scale)


def query_group(p: dict, qg: np.ndarray, keys: np.ndarray, vals: np.ndarray, L: int, t: int,
               summ, kc: np.ndarray, vc: np.ndarray, gates: np.ndarray | None):
    """All branches for one query position t of one GQA group.

    qg [G][d]; keys/vals [L][d]; summ = (mu, so, n) over all NB blocks of [0, L).
    Returns (out [G][d], sel [k], shat over candidates, gap)."""
    mu, so, n = summ
    scale = p["scale"]
    # candidates: blocks whose keys all lie at positions <= t
    last = np.arange(len(n)) * BLOCK + n - 1
    cand = np.nonzero((last <= t))[0]
    G = qg.shape[0]
    k = p["top_k"]
    if len(cand) > 0:
        s = block_scores(qg, mu[cand], so[cand], n[cand], p["alpha"], scale, p["so_kind"], p.get("P"))
        shat = group_scores(s)
        pick, gap = select_topk(shat, k)
        sel = np.array([cand[i] if i >= 0 else -1 for i in pick], dtype=np.int64)
    else:
        shat = np.zeros(0)
        sel = np.full(k, -1, dtype=np.int64)
        gap = np.inf
    out = np.zeros((G, keys.shape[1]))
    slc_pos = np.concatenate([np.arange(b * BLOCK, b * BLOCK + n[b]) for b in sel if b >= 0]) \
        if (sel >= 0).any() else np.zeros(0, dtype=np.int64)
    W = p["window"]
    win_pos = np.arange(max(0, t - W + 1), t + 1) if W > 0 else np.zeros(0, dtype=np.int64)
    if p["cmp_len"] > 0:
        j = np.arange(kc.shape[0])
        cmp_idx = j[j * p["cmp_stride"] + p["cmp_len"] - 1 <= t]
    else:
        cmp_idx = np.zeros(0, dtype=np.int64)
    for h in range(G):
        o_slc = softmax_attend(qg[h], keys[slc_pos], vals[slc_pos], scale)
        o_win = softmax_attend(qg[h], keys[win_pos], vals[win_pos], scale)
        o_cmp = softmax_attend(qg[h], kc[cmp_idx], vc[cmp_idx], scale)
        g = gates[h] if gates is not None else np.array([0.0, 1.0, 0.0])
        out[h] = g[0] * o_cmp + g[1] * o_slc + g[2] * o_win
    return out, sel, shat, gap


def params_of(w, scale: float | None = None, alpha: float | None = None) -> dict:
    """Method parameters of a synthetic workload description."""
    return {"top_k": w.top_k, "window": w.window, "cmp_len": w.cmp_len,
            "cmp_stride": w.cmp_stride, "so_kind": w.so_kind, "rank": w.rank,
            "alpha": w.alpha if alpha is None else alpha,
            "scale": (1.0 / np.sqrt(w.head_dim)) if scale is None else scale}


def build_unit(p: dict, keys: np.ndarray, vals: np.ndarray, L: int):
    """Summaries and compressed tokens of one (sequence, kv-head)."""
    summ = summaries(keys[:L], L, p["so_kind"], p["rank"], p.get("P"))
    if p["cmp_len"] > 0:
        kc = compressed_tokens(keys, L, p["cmp_len"], p["cmp_stride"])
        vc = compressed_tokens(vals, L, p["cmp_len"], p["cmp_stride"])
    else:
        kc = vc = np.zeros((0, keys.shape[1]))
    return summ, kc, vc


def run(inputs: dict, p: dict, seqs=None, groups=None, tokens=None):
    """Oracle over a batch (decode: t = L-1; prefill: t = q_pos0 + i).  When the
    inputs carry query subspaces P [H_kv][s][d], group g scores with P[g].

    Returns a dict keyed by (seq, group, token) with out [G][d], sel [k],
    shat (over candidates), gap; only the requested subsets are computed."""
    w = inputs["workload"]
    B, Hkv, G = w.batch, w.n_kv_heads, w.group
    seqs = range(B) if seqs is None else seqs
    groups = range(Hkv) if groups is None else groups
    res = {}
    subspace = inputs.get("P")                  # [H_kv][s][d] query subspaces, or None
    for s in seqs:
        L = int(inputs["lens"][s])
        for g in groups:
            pg = p if subspace is None else dict(p, P=np.asarray(subspace[g], dtype=np.float64))
            keys = inputs["K"][s, g, :L].astype(np.float64)
            vals = inputs["V"][s, g, :L].astype(np.float64)
            summ, kc, vc = build_unit(pg, keys, vals, L)
            toks = range(w.n_q_tokens) if tokens is None else tokens
            for i in toks:
                t = (w.q_pos0 + i) if w.prefill else L - 1
                qg = inputs["Q"][s, i, g * G:(g + 1) * G].astype(np.float64)
                gt = inputs["gates"][s, i, g * G:(g + 1) * G].astype(np.float64) \
                    if inputs["gates"] is not None else None
                res[(s, g, i)] = query_group(pg, qg, keys, vals, L, t, summ, kc, vc, gt)
    return res


def exact_group_scores(p: dict, qg: np.ndarray, keys: np.ndarray, L: int, t: int):
    """Group scores of the candidate blocks from exact masses ln m_b instead of the
    cumulant estimate ([COBS] 2.1: ranking by exact mass needs every key).
    Returns (candidate block indices, shat over them)."""
    n = block_sizes(L)
    last = np.arange(len(n)) * BLOCK + n - 1
    cand = np.nonzero(last <= t)[0]
    s = np.array([[np.log(attention_mass(qg[h], keys[b * BLOCK: b * BLOCK + n[b]], p["scale"]))
                   for b in cand] for h in range(qg.shape[0])])
    return cand, group_scores(s)


def oracle_selection_mass(p: dict, qg: np.ndarray, keys: np.ndarray, L: int, t: int) -> np.ndarray:
    """OSA: the group ranking on exact masses.  Returns the top-k candidate blocks
    (ascending, -1 padded)."""
    cand, shat = exact_group_scores(p, qg, keys, L, t)
    pick, _ = select_topk(shat, p["top_k"])
    return np.array([cand[i] if i >= 0 else -1 for i in pick], dtype=np.int64)
