"""Block-sparse masked ("Splash") attention forward for AMD MI355X (gfx950).

The computation lives in libsplash.so (hand-written HIP kernels behind a C
ABI, declared in include/splash.h); ``binding`` marshals torch tensors into
it, and ``autograd`` chains the forward and backward calls into one
differentiable function. ``workloads`` holds the seeded synthetic inputs.
"""

from .binding import (  # noqa: F401
    MaskInfo,
    SplashError,
    dense_mask_info_build,
    dense_mask_info_build_dkv,
    load_library,
    mask_info_build,
    mask_info_build_dkv,
    pointwise_bwd,
    pointwise_fwd,
    softmax_bwd,
    softmax_bwd_preprocess,
    splash_fwd,
    splash_fwd_lse,
)
from .autograd import splash_attention  # noqa: F401
from .workloads import CAUSAL, FULL, local_causal  # noqa: F401
