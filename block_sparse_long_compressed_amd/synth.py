"""Seeded synthetic workloads for block-sparse decode and prefill.

This module draws random inputs and nothing else: it holds no step of the
attention method (no block statistics, no scores, no selection, no softmax).
The fp64 oracle and the GPU path both consume exactly the arrays made here.

Key distribution (a stand-in for the long-context retrieval suite the COBS
paper evaluates on, which is not reproduced): every 64-key block b of every
(sequence, kv-head) has its own centre m_b ~ N(0, 0.1^2 I) and its own spread
sigma_b, log-uniform in [0.1, 2]; its keys are m_b + sigma_b * z with
z ~ N(0, I).  Blocks therefore differ mainly in spread, which is the case the
COBS explainer's "bundle A vs bundle B" picture is about (tight versus spread
bundles with the same centre).  A few "needle" keys equal 3*q/|q| for one
query head, so that head's logit on the needle is about 3.
Values, queries ~ N(0, 1); gates ~ U(0, 1).

bf16 workloads round Q, K and V to bfloat16 with round-to-nearest-even; the
arrays are returned as float32 holding bf16-exact values, so widening them to
fp64 (oracle) or narrowing them to torch.bfloat16 (GPU) is exact on both sides.

Draw order (fixed, part of the recipe): sequence lengths, Q, gates, then for
each (sequence, kv-head) in row-major order: block centres, block spreads,
unit normals for the keys; then V for all (sequence, kv-head); then needles.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

BLOCK = 64


@dataclass(frozen=True)
class Workload:
    """Shape and structure of one synthetic workload."""
    name: str
    batch: int
    max_len: int            # KV positions per sequence (upper bound)
    min_len: int            # lengths ~ U{min_len..max_len}; equal -> fixed
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    top_k: int
    window: int             # 0 = no sliding-window branch
    cmp_len: int            # 0 = no compressed branch
    cmp_stride: int
    so_kind: str            # 'diag' | 'lowrank' | 'lowrank_fp4' (bf16 mean, MX FP4 vectors)
    rank: int               # eigenpairs kept by the low-rank kinds
    alpha: float            # weight of the second-order term
    dtype: str              # 'bf16' | 'f32'
    needles: int            # planted needle keys per (sequence, kv-head)
    n_q_tokens: int = 1     # 1 = decode at t = L-1; >1 = prefill chunk
    q_pos0: int = -1        # prefill: position of the first query token
    gates: bool = True      # False -> only the selected-block branch (gates 0,1,0)
    subspace: int = 0       # query-subspace dimension s of the low-rank kinds (0 = off)
    n_calib: int = 512      # calibration query tokens drawn when subspace > 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def prefill(self) -> bool:
        return self.n_q_tokens > 1 or self.q_pos0 >= 0

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 query, 1 head, d=64, fp32, 1024 keys in 16 blocks, top-4, selected-block branch only.
    "tiny_f32_L1k": Workload("tiny_f32_L1k", 1, 1024, 1024, 1, 1, 64, 4, 0, 0, 16,
                             "diag", 0, 1.0, "f32", 1, gates=False),
    # batch 1, 32k keys, 64 q-heads / 4 kv-heads, d=128, bf16, top-16, window 512, pool 32/16.
    "decode_b1_L32k": Workload("decode_b1_L32k", 1, 32768, 32768, 64, 4, 128, 16, 512, 32, 16,
                               "diag", 0, 1.0, "bf16", 8),
    # batch 32, lengths U{16k..32k}, otherwise as the batch-1 decode.
    "decode_b32_L16k32k": Workload("decode_b32_L16k32k", 32, 32768, 16384, 64, 4, 128, 16, 512,
                                   32, 16, "diag", 0, 1.0, "bf16", 8),
    # one sequence of 32k keys, queries at positions 24576..32767.
    "prefill_T8k_L32k": Workload("prefill_T8k_L32k", 1, 32768, 32768, 64, 4, 128, 16, 512, 32,
                                 16, "diag", 0, 1.0, "bf16", 8, n_q_tokens=8192, q_pos0=24576),
    # batch 8, 128k keys, 32 q-heads / 8 kv-heads, top-32, window 1024, rank-4 summaries.
    "decode_b8_L128k_rank4": Workload("decode_b8_L128k_rank4", 8, 131072, 131072, 32, 8, 128, 32,
                                      1024, 32, 16, "lowrank", 4, 1.0, "bf16", 16),
    # the same with the compressed summary storage (bf16 mean, MX FP4 eigenvectors).
    "decode_b8_L128k_rank4_fp4": Workload("decode_b8_L128k_rank4_fp4", 8, 131072, 131072, 32, 8, 128,
                                          32, 1024, 32, 16, "lowrank_fp4", 4, 1.0, "bf16", 16),
    # the same with the rank-4 FP4 vectors in an 85-dimensional query subspace.
    "decode_b8_L128k_sub85_fp4": Workload("decode_b8_L128k_sub85_fp4", 8, 131072, 131072, 32, 8, 128,
                                          32, 1024, 32, 16, "lowrank_fp4", 4, 1.0, "bf16", 16, subspace=85),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), in place.

    Returns the same float32 array, now holding bf16-exact values."""
    assert x.dtype == np.float32
    flat = x.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        b = flat[s:s + step].view(np.uint32)
        lsb = (b >> np.uint32(16)) & np.uint32(1)
        b += np.uint32(0x7FFF) + lsb
        b &= np.uint32(0xFFFF0000)
    return x


def seq_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.min_len == w.max_len:
        return np.full(w.batch, w.max_len, dtype=np.int32)
    return rng.integers(w.min_len, w.max_len + 1, size=w.batch).astype(np.int32)


def make_inputs(w: Workload, seed: int, lens: Optional[np.ndarray] = None) -> dict:
    """Draw one seeded batch.

    Returns float32 arrays (bf16-exact for bf16 workloads):
      Q      [B][T][Hq][d]   (T = n_q_tokens)
      K, V   [B][Hkv][max_len][d], zero beyond each sequence's length
      gates  [B][T][Hq][3] in order (compressed, selected, window), or None
      lens   [B] int32
      needles list of (seq, kv_head, position, q_head, token)
      Qcal   [n_calib][Hq][d] calibration queries, or None   (subspace > 0)
      P      [Hkv][s][d] seeded orthonormal rows, or None     (subspace > 0)
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hq, Hkv, d, Lm = w.batch, w.n_q_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_len
    G = w.group
    if lens is None:
        lens = seq_lens(w, rng)
    lens = np.asarray(lens, dtype=np.int32)
    assert lens.shape == (B,) and int(lens.max()) <= Lm and int(lens.min()) >= 1

    Q = rng.standard_normal((B, T, Hq, d), dtype=np.float32)
    gates = rng.uniform(0.0, 1.0, size=(B, T, Hq, 3)).astype(np.float32) if w.gates else None

    K = np.zeros((B, Hkv, Lm, d), dtype=np.float32)
    lo, hi = math.log(0.1), math.log(2.0)
    for s in range(B):
        L = int(lens[s])
        nb = -(-L // BLOCK)
        for h in range(Hkv):
            centre = rng.normal(0.0, 0.1, size=(nb, 1, d)).astype(np.float32)
            spread = np.exp(rng.uniform(lo, hi, size=(nb, 1, 1))).astype(np.float32)
            z = rng.standard_normal((nb, BLOCK, d), dtype=np.float32)
            keys = (centre + spread * z).reshape(nb * BLOCK, d)
            K[s, h, :L] = keys[:L]

    V = rng.standard_normal((B, Hkv, Lm, d), dtype=np.float32)
    for s in range(B):
        V[s, :, int(lens[s]):] = 0.0

    Qcal = P = None
    if w.subspace:
        # Queries of each kv-head group concentrated near an s-dimensional subspace:
        # q = U_h diag(sigma) z with a random orthonormal U_h and sigma_j proportional
        # to exp(-2j/s) (98% of E|q|^2 in the first s directions), scaled to E|q|^2 = d.
        # Calibration tokens come from the same distribution.  P is a seeded random
        # orthonormal [s][d] per kv-head, an input the parity tests hand to both sides.
        sig = np.exp(-2.0 * np.arange(d) / w.subspace)
        sig *= math.sqrt(d / float((sig * sig).sum()))
        Qcal = rng.standard_normal((w.n_calib, Hq, d)).astype(np.float32)
        P = np.zeros((Hkv, w.subspace, d), dtype=np.float32)
        for h in range(Hkv):
            U = np.linalg.qr(rng.standard_normal((d, d)))[0]
            hs = slice(h * G, (h + 1) * G)
            Q[:, :, hs] = ((Q[:, :, hs].astype(np.float64) * sig) @ U.T).astype(np.float32)
            Qcal[:, hs] = ((Qcal[:, hs].astype(np.float64) * sig) @ U.T).astype(np.float32)
            P[h] = np.linalg.qr(rng.standard_normal((d, w.subspace)))[0].T.astype(np.float32)
        if w.dtype == "bf16":
            round_bf16(Qcal)

    if w.dtype == "bf16":
        round_bf16(Q)
        # needle direction is taken from the bf16 query so it is exact on both sides
    needles = []
    for s in range(B):
        L = int(lens[s])
        nb = -(-L // BLOCK)
        for h in range(Hkv):
            cnt = min(w.needles, nb)
            blocks = rng.choice(nb, size=cnt, replace=False)
            for b in blocks:
                nbk = min(BLOCK, L - int(b) * BLOCK)
                pos = int(b) * BLOCK + int(rng.integers(0, nbk))
                qh = h * G + int(rng.integers(0, G))
                tok = int(rng.integers(0, T))
                q = Q[s, tok, qh].astype(np.float64)
                K[s, h, pos] = (3.0 * q / np.linalg.norm(q)).astype(np.float32)
                needles.append((s, h, pos, qh, tok))

    if w.dtype == "bf16":
        round_bf16(K)
        round_bf16(V)
    return {"Q": Q, "K": K, "V": V, "gates": gates, "lens": lens, "needles": needles,
            "workload": w, "seed": seed, "Qcal": Qcal, "P": P}

