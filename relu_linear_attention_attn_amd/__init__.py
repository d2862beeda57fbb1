"""ReLU linear self-attention (Sana Linear DiT) for AMD MI355X: forward (non-causal,
block-causal and token-causal, ReLU or another feature map; also from the QKV projection, with the
state formed in the projection's epilogue) and backward.

The compute runs in hand-written HIP kernels behind a C ABI
(``libsana_linattn.so``, declared in ``include/sana_linattn.h``); this package
is a thin ctypes binding plus the seeded workload generator. The library is
loaded on first use and every call raises if it has not been built.
"""
from .binding import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    FMAPS,
    VARIANT_AUTO,
    VARIANT_FUSED,
    VARIANT_SPLIT,
    SanaError,
    apply,
    backward,
    block_causal_workspace_size,
    bwd_workspace_size,
    causal_workspace_size,
    forward,
    forward_block_causal,
    forward_causal,
    forward_fmap,
    forward_noalloc,
    forward_profiled,
    forward_qkv,
    forward_strided,
    kv_state,
    lib,
    qkv_workspace_size,
    state_size,
    strerror,
    workspace_size,
)
