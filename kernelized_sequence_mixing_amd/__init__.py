"""Kernelized linear attention for AMD MI355X (gfx950).

    o_i = phi(q_i)^T S / (phi(q_i)^T z + eps),  S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j)

non-causal and causal (optionally with a fixed decay or a per-step diagonal
gate), plus the recurrent decode step, with elu+1 or FAVOR+ feature maps. The
work runs in the HIP kernels of ``liblinattn.so`` behind the C ABI declared in
``include/linattn.h``; this package only marshals torch tensors into it.
"""
from ._native import LinattnError, LIB_PATH  # noqa: F401
from .api import forward, decode_step, feature_map, workspace_size, segments  # noqa: F401
from .api import PreparedForward, PreparedDecode, backward, PreparedBackward  # noqa: F401
from .api import forward_batch, PreparedForwardBatch, launch_times  # noqa: F401
from .api import forward_noalloc, softmax_attention, PreparedSoftmax  # noqa: F401

__all__ = ["forward", "forward_batch", "PreparedForwardBatch", "backward", "decode_step", "feature_map", "workspace_size", "segments", "PreparedForward",
           "PreparedBackward", "PreparedDecode", "launch_times", "forward_noalloc", "softmax_attention", "PreparedSoftmax",
           "LinattnError", "LIB_PATH"]
