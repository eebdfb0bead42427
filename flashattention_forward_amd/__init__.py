"""MI355X (gfx950) FlashAttention: C-ABI library + thin binding.

The compute path is libattn_mi355x.so (hand-written HIP kernels for the
forward pass, its split-KV decode and quantised variants, and the backward
pass); this package only marshals torch tensors into its C entry points.
"""
from .binding import (  # noqa: F401
    ATTN_BF16, ATTN_FP16, attn_bwd, attn_bwd_varlen, attn_fwd, attn_fwd_decode, attn_fwd_exp2_split, debug_exp2_poly, attn_fwd_fp4p, attn_fwd_fp8, attn_fwd_i8, attn_fwd_q8,
    attn_fwd_varlen, build_info, debug_cvt_e2m1, debug_cvt_e4m3, debug_qk_f8, debug_qk_i32, decode_splits, lib, quantize_rows_i8,
    quantize_tensor_e4m3, quantize_tensor_i8, rotate_quantize_e4m3, status_str, workspace_bytes,
)
