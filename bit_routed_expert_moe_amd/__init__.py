"""MI355X (gfx950) routed-expert MoE decode layer.

The compute lives in ``libmoe_layer.so`` (hand-written HIP kernels behind a C
ABI, see include/moe_layer.h).  This package only marshals torch tensors into
that ABI; there is no Python or CPU fallback for any step.
"""
from .layer import (  # noqa: F401
    KernelTimer, Layer, MoeError, MOE_BF16, MOE_F32, lib, record_bytes, stack_forward, stream_read,
)
