"""Fused exact attention (FlashAttention-2 style) for AMD MI355X / gfx950.

The compute lives in libflashattn.so (hand-written HIP, C ABI in include/flash_attn.h);
this package is its thin Python binding.  Build with
`python -m online_softmax_fwd_flash_amd.build`.
"""
from .api import (FlashAttnError, flash_attn_fwd, flash_attn_bwd, flash_attn_bwd_noalloc,
                  flash_attn_bwd_preprocess,
                  flash_attn_bwd_dkdv, flash_attn_bwd_dq, flash_attn_bwd_dq_dvec,
                  flash_attn_fwd_strided, flash_attn_bwd_strided, flash_attn_bwd_grad16,
                  flash_attn_qk_norm_rope,
                  flash_attn_block_class, flash_attn_block_class_qk, flash_attn_kv_block_range_qk,
                  flash_attn_kv_block_range, flash_attn_default_tiles, flash_attn_check_layout,
                  flash_attn_version, flash_attn_mfma_rate_probe)
from ._lib import LIB_PATH, EXPORTS

__all__ = ["FlashAttnError", "flash_attn_fwd", "flash_attn_bwd", "flash_attn_bwd_noalloc",
           "flash_attn_bwd_preprocess",
           "flash_attn_bwd_dkdv", "flash_attn_bwd_dq", "flash_attn_bwd_dq_dvec",
           "flash_attn_fwd_strided", "flash_attn_bwd_strided", "flash_attn_bwd_grad16",
           "flash_attn_qk_norm_rope",
           "flash_attn_block_class", "flash_attn_block_class_qk", "flash_attn_kv_block_range_qk",
           "flash_attn_kv_block_range", "flash_attn_default_tiles", "flash_attn_check_layout",
           "flash_attn_version", "flash_attn_mfma_rate_probe",
           "LIB_PATH", "EXPORTS"]
