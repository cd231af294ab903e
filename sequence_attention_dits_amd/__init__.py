"""One rank's share of context-parallel attention (Ulysses, Ulysses
Anything, Ring, Unified) on AMD Instinct MI355X (gfx950).

The work runs in libuaa.so (hand-written HIP kernels behind a C ABI,
include/uaa.h); this package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    UAA_BF16,
    UAA_ERR_HIP,
    UAA_ERR_INVALID_ARG,
    UAA_ERR_UNSUPPORTED,
    UAA_FP32,
    UAA_HEAD2SEQ,
    UAA_MAX_WORLD,
    UAA_OK,
    UAA_SEQ2HEAD,
    USP_MASK_CAUSAL,
    USP_MASK_FULL,
    USP_MASK_STRIPE,
    USP_MASK_ZIGZAG,
    USP_MAX_PARTS,
    LIB_PATH,
    UaaError,
    lib,
    mask_causal,
    mask_full,
    mask_stripe,
    mask_zigzag,
    attn_workspace,
    usp_attn_fwd_lse,
    usp_attn_fwd_lse_gather,
    usp_attn_bwd,
    usp_attn_bwd_delta,
    usp_lse_merge,
    usp_mask,
    uaa_seq2head_permute,
    uaa_seq2head_permute_multi,
    UAA_MAX_PERMUTE_TENSORS,
)
