"""Exact attention forward (FlashAttention-2 style) for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(`exact_attention_49_amd/csrc`, declared in `include/exact_attn.h`); `attn_fwd` and
`attn_fwd_varlen` below are thin ctypes bindings that marshal torch device tensors and the
current HIP stream into it.  The library is loaded on first use and its absence is an error.
"""

from .binding import (AttnError, attn_fwd, attn_fwd_varlen, library_path,  # noqa: F401
                      load_library)

__all__ = ["AttnError", "attn_fwd", "attn_fwd_varlen", "library_path", "load_library"]
