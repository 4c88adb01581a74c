"""MI355X-native forward pass of a DeepSpeed-MoE-style MoE FFN layer.

The layer runs in libmoe_mi355x.so (hand-written HIP kernels for gfx950, C ABI
in include/moe.h); `binding` is its ctypes wrapper and `workloads` the seeded
synthetic inputs. Importing this package loads nothing; the first binding call
loads the library and fails loudly if it has not been built.
"""
__all__ = ["binding", "workloads"]
