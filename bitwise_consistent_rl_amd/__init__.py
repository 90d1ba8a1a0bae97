"""Batch-invariant logprob recompute for MI355X (gfx950).

libbci.so (HIP kernels + C ABI, include/bci.h) does all device work; this
package holds its ctypes binding (``_abi``), the in-tree build step
(``build``) and the host-side drivers (``engine``: packed recompute,
op-by-op recompute, continuous-batching rollout, acceptance statistics).
Importing the package does not load the library; the first call does, and
fails loudly if it is not built.
"""
__all__ = ["build", "engine", "_abi"]
