"""MI355X-native trainable MoE expert layer (forward and backward on one GPU).

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP kernels
for gfx950); :mod:`grouped_gemm_02_amd.binding` marshals torch tensors into its
entry points. Importing this package loads nothing: the library is loaded on
first use and a missing library is an error, never a fallback.
"""
__all__ = ["binding", "inputs"]
