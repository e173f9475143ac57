"""Blockwise causal varlen attention for MI355X (gfx950).

The compute lives in a HIP shared library with a C ABI (``include/attn.h``);
``blockwise_causal_varlen_amd.lib`` is the thin ctypes binding over it and
``blockwise_causal_varlen_amd.inputs`` draws the seeded synthetic workloads.
Importing the package does not load the library; the binding loads it on first
use and raises if it has not been built.
"""

__all__ = ["lib", "inputs"]
