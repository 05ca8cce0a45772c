"""Fused single-pass attention KL divergence KL(P1 || P2) for AMD MI355X.

The computation lives in the HIP library libstreamkl.so (C ABI in
include/streamkl.h); this package only loads it and marshals torch tensors.
"""
from .ops import bwd, bwd_both, bwd_select, fwd, fwd_auto, fwd_splitk, splitk_auto, splitk_workspace_bytes  # noqa: F401
from .autograd import attention_kl  # noqa: F401
