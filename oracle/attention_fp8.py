"""Plain CPU oracle for the FP8 attention forward (fp64).

TEST INFRASTRUCTURE ONLY, like oracle/attention.py: nothing on the product path may import,
call or run it.  It shares no code with the HIP kernels or their host library.

What it computes.  Q, K and V arrive as 8-bit floats (E4M3) with one fp32 descale factor per
tensor; the values they stand for are code * descale.  The pages fold the Q and K descales
into the softmax scale and keep the V descale for the output (page "flash_fwd_kernel.h"
@c272619, `compute_attn_ws_fp8`: softmax_scale_log2 * descale_q * descale_k, and descale_v;
page "flash_fwd_kernel.h" @26a6e0a: q_scale * k_scale multiply softmax_scale_log2, a missing
scale pointer meaning 1).  The exact result of that is plain attention of the dequantized
tensors,

    O = softmax(scale * (dq Q8) (dk K8)^T + mask) (dv V8),  LSE over the same scores,

so the oracle decodes the codes by the E4M3 definition, multiplies by the descales in float64
and calls the forward oracle's definition.  How the kernels round P on the way (to E4M3, with
the pages' offset of 8 in the exponent, `Max_offset`) is a property of the kernels; it is
accounted for in the tests' error bound, not here.

E4M3 (the OCP 8-bit format with 4 exponent bits, bias 7, and 3 mantissa bits, no infinities):
bit 7 is the sign; exponent field e = bits 6..3 and mantissa m = bits 2..0 give
(-1)^s * 2^(e-7) * (1 + m/8) for e >= 1 and (-1)^s * 2^-6 * (m/8) for e = 0 (subnormals);
the codes with e = 15 and m = 7 are NaN.  The largest finite magnitude is 448.

Pinned by tests under tests/ (the decode against torch's float8_e4m3fn conversion for all 256
codes and hand-worked codes; the attention part is the forward oracle, pinned on its own).
"""

from __future__ import annotations

import numpy as np

from .attention import attention_dense, attention_varlen

__all__ = ["decode_e4m3", "attention_fp8_dense", "attention_fp8_varlen", "E4M3_MAX"]

E4M3_MAX = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """Float64 values of E4M3 codes (any integer array of bytes), by the format's definition."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.exp2(e.astype(np.float64) - 7.0) * (1.0 + m / 8.0)
    sub = sign * np.exp2(-6.0) * (m / 8.0)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def _descale(x, d) -> float:
    return 1.0 if d is None else float(np.float32(d))


def attention_fp8_dense(q8, k8, v8, scale: float, descale_q=None, descale_k=None,
                        descale_v=None, causal: bool = False, window_left: int = -1,
                        window_right: int = -1):
    """q8 [B, H, N, d], k8, v8 [B, Hkv, N, d] as E4M3 codes (uint8); descales are fp32
    scalars or None (= 1).  Returns (O, LSE) float64 of the dequantized problem."""
    q = decode_e4m3(q8) * _descale(q8, descale_q)
    k = decode_e4m3(k8) * _descale(k8, descale_k)
    v = decode_e4m3(v8) * _descale(v8, descale_v)
    return attention_dense(q, k, v, scale, causal, window_left, window_right)


def attention_fp8_varlen(q8, k8, v8, cu_seqlens, scale: float, descale_q=None,
                         descale_k=None, descale_v=None, causal: bool = False,
                         window_left: int = -1, window_right: int = -1):
    """Packed batch: q8 [H, total, d], k8, v8 [Hkv, total, d] E4M3 codes."""
    q = decode_e4m3(q8) * _descale(q8, descale_q)
    k = decode_e4m3(k8) * _descale(k8, descale_k)
    v = decode_e4m3(v8) * _descale(v8, descale_v)
    return attention_varlen(q, k, v, cu_seqlens, scale, causal, window_left, window_right)
