"""Single-GPU fused MoE layer forward for MI355X (gfx950).

The compute path is libmoe.so (C ABI in include/moe.h, HIP kernels under
csrc/); ``binding`` marshals torch tensors into it.  Importing this package
does not load the library; the first call does, and fails loudly if it has
not been built.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
