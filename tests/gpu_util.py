"""Shared helpers of the GPU parity tests: the device-side helpers of the package
(upload, build, decode, prefill) and the checks of GPU results against the oracle."""
from __future__ import annotations

import numpy as np

from block_sparse_long_compressed_amd import binding as B  # noqa: F401
from block_sparse_long_compressed_amd.runtime import (SO_KINDS, build, decode, params_for,  # noqa: F401
                                                      prefill, to_device)

GAP = 1e-3          # score gap (natural-log units) below which several selections are correct


def selection_ok(sel_gpu: np.ndarray, shat: np.ndarray, k: int, cand_offset: int = 0):
    """Is the GPU selection one of the correct top-k sets of the oracle scores shat
    (over candidate blocks 0..len(shat)-1)?  Returns (ok, message)."""
    nc = len(shat)
    take = min(k, nc)
    chosen = [int(b) for b in sel_gpu if b >= 0]
    if list(sel_gpu[take:]) != [-1] * (k - take):
        return False, f"padding wrong: {sel_gpu}"
    if len(chosen) != take or chosen != sorted(chosen) or len(set(chosen)) != take:
        return False, f"not {take} ascending distinct blocks: {sel_gpu}"
    if take == 0:
        return True, ""
    if max(chosen) >= nc:
        return False, f"non-candidate selected: {chosen} (candidates {nc})"
    order = sorted(range(nc), key=lambda b: (-shat[b], b))
    sk = shat[order[take - 1]]
    sk1 = shat[order[take]] if take < nc else -np.inf
    sure_in = {b for b in range(nc) if shat[b] - sk1 >= GAP}
    sure_out = {b for b in range(nc) if sk - shat[b] >= GAP}
    S = set(chosen)
    if not sure_in <= S:
        return False, f"missing sure blocks {sorted(sure_in - S)}"
    if S & sure_out:
        return False, f"selected excluded blocks {sorted(S & sure_out)}"
    return True, ""


def rel_err_rows(a: np.ndarray, b: np.ndarray) -> float:
    """Largest per-row relative L2 error of a against reference b."""
    num = np.linalg.norm(a - b, axis=-1)
    den = np.maximum(np.linalg.norm(b, axis=-1), 1e-30)
    return float((num / den).max())


def bf16_round64(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of fp64 values, returned as fp64."""
    f = x.astype(np.float32)
    # fp64 -> fp32 rounding first cannot create a double rounding error large enough to
    # matter at the +-1 ulp bar used by the callers
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)
