"""Absorbed MLA attention over a 512-wide bf16 latent KV cache, for AMD MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(`libmla_absorb.so`, declared in include/mla_absorb.h).  The Python side only
marshals arguments: `binding` exposes the library calls with the same names and
takes torch tensors for device memory and the current HIP stream.

Importing this package loads nothing; `binding.lib()` loads the library and
raises if it is missing.
"""
__all__ = ["binding", "workloads"]
