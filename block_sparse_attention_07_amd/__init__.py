"""Block-sparse video-DiT self-attention for AMD MI355X (gfx950).

    out = sparse_attn(q, k, v, mask_bits, scale)

computes softmax(scale * Q K^T + M) V where M is 0 on the 64x64 blocks whose bit
is set in the per-head packed row mask and -inf elsewhere (ScalingAttention,
section 4.3.2); ``sparse_attn_b128`` takes ScalingAttention's own format, 128x128 blocks
in 32-bit words.  Mask producers: ``mask_from_stripes`` (PSA stripe tuples),
``block_scores_meanpool`` + ``mask_from_block_scores_topp`` (online top-p with a
top-k minimum), ``mask_from_threshold_map`` (static masks M = I(T <= p*)) with
``threshold_map_resize`` / ``mask_resize`` for other resolutions, and
``hilbert3d_order`` + ``permute_tokens`` for Hilbert-ordered tokens;
``attn_fidelity`` measures how far a mask moves attention rows (Hellinger
distance, ScalingAttention Eqs. 3-4).  All compute runs in the HIP library ``libbsattn.so``; this package only
marshals arguments.
"""
from .api import (  # noqa: F401
    BLOCK,
    attn_fidelity,
    block_scores_meanpool,
    hilbert3d_order,
    mask_b128_to_b64,
    mask_from_block_scores_topp,
    mask_from_stripes,
    mask_from_threshold_map,
    mask_resize,
    mask_words,
    mfma_probe,
    permute_tokens,
    plan,
    sparse_attn,
    sparse_attn_b128,
    sparse_attn_noalloc,
    threshold_map_resize,
    workspace_bytes,
)
from ._lib import BsaError, LIB_PATH  # noqa: F401
