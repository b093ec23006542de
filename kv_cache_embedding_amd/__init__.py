"""TurboQuant quantize / inner-product path on MI355X (gfx950).

A thin binding over the C ABI of ``libtq.so`` (declared in ``include/tq.h``): every
function here has the name of the C call it wraps, turns torch tensors into raw device
pointers and sizes, passes torch's current HIP stream, and raises ``TQError`` on a non-zero
status.  All arithmetic runs in the HIP kernels; there is no CPU fallback.  Importing
this package does not load the library; the first call does, and fails loudly if it is
missing.
"""
from ._binding import (  # noqa: F401
    TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP, TQ_EWORKSPACE, TQ_F32, TQ_BF16, TQ_EST_PROD,
    TQ_EST_MSE, TQError, lib_path, load_library, tq_codebook_build, tq_codebook_build_sphere,
    tq_params_bytes, tq_prepare, tq_prepare_orthogonal_qjl, tq_quantize_split, tq_score_split_ws_bytes,
    tq_score_ip_split, tq_score_split_prepare, tq_score_ip_split_prepared, tq_quantize_mse_split,
    tq_attention_split_ws_bytes, tq_attention_split, tq_quantize, tq_quantize_with_rotation, tq_quantize_mse, tq_append_ws_bytes, tq_append, tq_dequantize, tq_score_ws_bytes, tq_score_ip,
    tq_score_ip_noalloc, tq_score_noalloc_max_ws_bytes, tq_score_prepare, tq_score_ip_prepared,
    tq_attention_ws_bytes, tq_attention, tq_topk_ws_bytes, tq_topk, tq_last_error,
)

__all__ = [
    "TQ_OK", "TQ_EINVAL", "TQ_EUNSUPPORTED", "TQ_EHIP", "TQ_EWORKSPACE", "TQ_F32", "TQ_BF16",
    "TQ_EST_PROD", "TQ_EST_MSE", "TQError", "lib_path", "load_library", "tq_codebook_build",
    "tq_codebook_build_sphere", "tq_params_bytes", "tq_prepare", "tq_prepare_orthogonal_qjl",
    "tq_quantize_split", "tq_score_split_ws_bytes", "tq_score_ip_split", "tq_score_split_prepare",
    "tq_score_ip_split_prepared", "tq_quantize_mse_split",
    "tq_attention_split_ws_bytes", "tq_attention_split", "tq_quantize", "tq_quantize_with_rotation", "tq_quantize_mse", "tq_append_ws_bytes", "tq_append",
    "tq_dequantize",
    "tq_score_ws_bytes", "tq_score_ip", "tq_score_ip_noalloc", "tq_score_noalloc_max_ws_bytes", "tq_score_prepare", "tq_score_ip_prepared", "tq_attention_ws_bytes", "tq_attention",
    "tq_topk_ws_bytes", "tq_topk", "tq_last_error",
]
