"""MI355X-native fused attention KL divergence (StreamKL) for PyTorch-ROCm.

The computation lives in libstreamkl.so (hand-written HIP kernels for
gfx950, C ABI in include/streamkl.h); this package is its thin binding.
"""
from .streamkl import (  # noqa: F401
    BWD_AUTO,
    BWD_DK_ONLY,
    BWD_DQ_ONLY,
    BWD_FUSED,
    BWD_SEPARATE,
    StreamKLError,
    attention_kl,
    attention_kl_loss,
    bwd_plan,
    bwd_workspace_bytes,
    fwd_plan,
    fwd_loss_workspace_bytes,
    fwd_workspace_bytes,
    library,
    make_shape,
    packed_shape_of,
    shape_of,
    streamkl_bwd,
    streamkl_bwd_joint,
    kl_loss,
    streamkl_fwd,
    streamkl_fwd_loss,
)
