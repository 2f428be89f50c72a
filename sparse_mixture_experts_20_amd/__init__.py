"""Sparse Mixture-of-Experts layer forward for AMD Instinct MI355X (gfx950).

The layer runs in hand-written HIP kernels behind a C ABI (``include/moe.h``,
``libmoe.so``); :mod:`.binding` marshals torch device tensors to it.
"""
__all__ = ["binding", "workloads"]
