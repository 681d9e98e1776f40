"""exact_tiled_attention_13_amd -- exact tiled softmax attention on MI355X (gfx950).

Python face of ``libfa_mi355x.so``: the same entry points as the C ABI in
``include/fa_mi355x.h``, taking torch tensors for device memory and the
current stream. The computation itself runs only in the library's HIP
kernels.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    FA_ERR_HIP,
    FA_ERR_INVALID_ARG,
    FA_ERR_UNSUPPORTED,
    FA_ERR_WORKSPACE,
    FA_NOALLOC_SCRATCH_BYTES,
    FA_OK,
    LIB_PATH,
    LIB_POISON_PATH,
    FaError,
    attn_bwd,
    attn_bwd_dkdv,
    attn_bwd_dq,
    attn_bwd_dq_prep,
    attn_bwd_gqa,
    attn_bwd_gqa_workspace_size,
    attn_bwd_noalloc,
    attn_bwd_prep,
    attn_bwd_workspace_size,
    attn_decode,
    attn_decode_workspace_size,
    attn_fwd,
    attn_fwd_fp32,
    attn_fwd_fp8,
    attn_fwd_gqa,
    default_scale,
    lib,
    status_string,
    use_library,
    workspace,
    workspace_gqa,
)
