"""COBS block-sparse attention for MI355X (gfx950).

The compute path is libcobs.so (hand-written HIP kernels behind a C ABI, see
include/cobs.h); `binding` marshals torch tensors into it.  `synth` draws the
seeded synthetic workloads.  Importing the package loads nothing; the library
is loaded on first use and its absence is an error.
"""
