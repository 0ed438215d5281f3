"""Sparse MoE layer forward for MI355X (gfx950): HIP kernels behind a C ABI.

``sparse_mixture_experts_amd.moe`` binds the C-ABI library (``libmoe_mi355x.so``)
with ctypes; ``sparse_mixture_experts_amd.inputs`` draws seeded synthetic layers.
Importing the package loads nothing; the library is loaded on first use and a
missing library is an error, never a silent fallback.
"""
__all__ = ["moe", "inputs"]
