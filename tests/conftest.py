import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# (sequence, kv-head) units of the 8 x 128k workloads checked at full size: two per
# sequence, every kv head twice
LONG_UNITS = [(b, (3 * b + j) % 8) for b in range(8) for j in (0, 4)]


@pytest.fixture(scope="session")
def long_inputs():
    """The 8 x 128k rank-4 workload's inputs (shared by its fp32 and compressed storages:
    the draws do not depend on the storage)."""
    from block_sparse_long_compressed_amd import synth
    w = synth.WORKLOADS["decode_b8_L128k_rank4"]
    print("[fixture] drawing the 8 x 128k inputs", flush=True)
    return w, synth.make_inputs(w, 4)


@pytest.fixture(scope="session")
def long_oracle_lowrank(long_inputs):
    """The oracle's fp64 rank-4 summaries and pooled tokens of LONG_UNITS."""
    import numpy as np
    from oracle import cobs_oracle as O
    w, x = long_inputs
    p = O.params_of(w)
    res = {}
    for (b, h) in LONG_UNITS:
        print(f"[fixture] oracle rank-4 summaries of unit ({b}, {h})", flush=True)
        L = int(x["lens"][b])
        res[(b, h)] = O.build_unit(p, x["K"][b, h, :L].astype(np.float64), x["V"][b, h, :L].astype(np.float64), L)
    return res
