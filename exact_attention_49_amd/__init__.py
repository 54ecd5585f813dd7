"""Exact attention (FlashAttention-2 style) for AMD Instinct MI355X (gfx950): the forward pass
and its backward.

The compute path is a C-ABI shared library of hand-written HIP kernels
(`exact_attention_49_amd/csrc`, declared in `include/exact_attn.h`).  The functions below
(`attn_fwd`, `attn_fwd_varlen`, their grouped-query, persistent, split-KV and FP8 variants, and
`attn_bwd`, `attn_bwd_varlen`) are thin ctypes bindings that marshal torch device tensors and
the current HIP stream into it.  The library is loaded on first use and its absence is an
error.
"""

from .binding import (AttnError, attn_bwd, attn_bwd_varlen, attn_fwd,  # noqa: F401
                      attn_fwd_fp8, attn_fwd_gqa, attn_fwd_persistent, attn_fwd_splitkv,
                      attn_fwd_splitkv_noalloc, attn_fwd_varlen, attn_fwd_varlen_fp8,
                      attn_fwd_varlen_gqa, attn_fwd_varlen_persistent, attn_fwd_varlen_splitkv,
                      bwd_workspace_size, library_path, load_library, splitkv_num_splits,
                      splitkv_workspace_size, varlen_bwd_workspace_size,
                      varlen_splitkv_num_splits, varlen_splitkv_workspace_size)

__all__ = ["AttnError", "attn_fwd", "attn_fwd_varlen", "attn_fwd_gqa", "attn_fwd_varlen_gqa",
           "attn_fwd_persistent", "attn_fwd_varlen_persistent", "attn_fwd_splitkv",
           "attn_fwd_splitkv_noalloc", "attn_fwd_varlen_splitkv", "splitkv_num_splits",
           "splitkv_workspace_size", "varlen_splitkv_num_splits",
           "varlen_splitkv_workspace_size", "attn_fwd_fp8", "attn_fwd_varlen_fp8", "attn_bwd",
           "attn_bwd_varlen", "bwd_workspace_size", "varlen_bwd_workspace_size",
           "library_path", "load_library"]
