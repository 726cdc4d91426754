"""MI355X-native greedy speculative verification through an MoE decoder.

The compute path is the C-ABI library ``libmoe_verify.so`` (HIP kernels for gfx950),
reached through :mod:`.binding`. Importing this package loads nothing; the binding
loads the library on first use and raises if it is missing.
"""
__all__ = ["workload", "binding"]
