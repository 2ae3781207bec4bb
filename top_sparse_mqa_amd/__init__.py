"""Top-k sparse multi-query attention (forward and backward) for AMD Instinct MI355X.

The computation runs in hand-written gfx950 HIP kernels behind the C ABI of
libsparse_mqa.so (include/sparse_mqa.h); this package is the Python binding.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    DkvSteps,
    SparseMQAError,
    bwd_dkv,
    bwd_dq,
    bwd_main,
    bwd_postprocess,
    bwd_workspace_bytes,
    bwd_dsink,
    bwd_preprocess,
    default_scale,
    load_library,
    sparse_mqa_bwd_interface,
    sparse_mqa_fwd_interface,
)
from .autograd import SparseMQAFunction, sparse_mqa  # noqa: F401
