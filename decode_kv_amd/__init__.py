"""decode_kv_amd: CSA2 hierarchical sparse-attention decode for MI355X (gfx950).

The hot path is a C-ABI shared library of hand-written HIP kernels
(``libcsa2.so``); :mod:`decode_kv_amd.csa2` is its thin ctypes binding,
:mod:`decode_kv_amd.pipeline` orders the calls of one decode step, and
:mod:`decode_kv_amd.inputs` / :mod:`decode_kv_amd.workloads` describe and
generate the seeded synthetic workloads.

Importing the package loads nothing; the binding loads the library on first
use and raises if it has not been built.
"""

__all__ = ["csa2", "inputs", "workloads", "pipeline"]
