"""ctypes binding of the C-ABI library declared in include/exact_attn.h.

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory (the tensors) and the current HIP stream.  There is no CPU
fallback: if the library is missing, or a tensor is not on the GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

__all__ = ["AttnError", "attn_fwd", "attn_fwd_varlen", "attn_fwd_gqa", "attn_fwd_varlen_gqa",
           "attn_fwd_persistent", "attn_fwd_varlen_persistent",
           "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc",
           "attn_fwd_varlen_splitkv", "splitkv_num_splits", "splitkv_workspace_size",
           "varlen_splitkv_num_splits", "varlen_splitkv_workspace_size", "attn_bwd",
           "attn_bwd_varlen", "bwd_workspace_size", "varlen_bwd_workspace_size", "attn_fwd_fp8",
           "attn_fwd_varlen_fp8", "library_path", "load_library", "STATUS", "EXPORTED_SYMBOLS"]

LIB_NAME = "libexact_attn.so"

DTYPE_CODES = {torch.float16: 0, torch.bfloat16: 1}

STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_INVALID_ARG",
    2: "ATTN_ERR_UNSUPPORTED_HEAD_DIM",
    3: "ATTN_ERR_UNSUPPORTED_DTYPE",
    4: "ATTN_ERR_MISALIGNED",
    5: "ATTN_ERR_TOO_LARGE",
    6: "ATTN_ERR_HIP",
    7: "ATTN_ERR_SCRATCH_LIMIT",
}

NOALLOC_SCRATCH_BYTES = 64 << 20   # ATTN_NOALLOC_SCRATCH_BYTES

# (name, restype, argtypes) for every function include/exact_attn.h declares
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
EXPORTED_SYMBOLS = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "attn_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                             _P]),
    "attn_fwd_gqa": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "attn_fwd_varlen_gqa": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                 _I, _I, _P]),
    "attn_fwd_persistent": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                                 _P]),
    "attn_fwd_varlen_persistent": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                        _F, _I, _I, _I, _P]),
    "attn_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I,
                              _P, _S, _P]),
    "attn_fwd_varlen_splitkv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                     _I, _I, _I, _I, _P, _S, _P]),
    "attn_fwd_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                                      _I, _I, _P]),
    "attn_fwd_splitkv_workspace_size": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_fwd_varlen_splitkv_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "attn_fwd_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "attn_fwd_varlen_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "attn_fwd_fp8": (_I, [_P] * 8 + [_I] * 6 + [_F] + [_I] * 3 + [_P]),
    "attn_fwd_varlen_fp8": (_I, [_P] * 9 + [_I] * 7 + [_F] + [_I] * 3 + [_P]),
    "attn_bwd": (_I, [_P] * 9 + [_I] * 6 + [_F] + [_I] * 3 + [_P, _S, _P]),
    "attn_bwd_varlen": (_I, [_P] * 10 + [_I] * 7 + [_F] + [_I] * 3 + [_P, _S, _P]),
    "attn_bwd_workspace_size": (_S, [_I, _I, _I]),
    "attn_bwd_varlen_workspace_size": (_S, [_I, _I]),
    "attn_device_info": (_I, [_I, _P, _P]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_last_hip_error": (_I, []),
}

_LIB = None
_LOCK = threading.Lock()


class AttnError(RuntimeError):
    """A non-zero status from the library (or a tensor it cannot take)."""

    def __init__(self, msg: str, status: int | None = None):
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)


def load_library():
    """Load the built HIP library once and declare its signatures."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            path = library_path()
            if not os.path.exists(path):
                raise AttnError(f"HIP library {path} is not built; run "
                                "python -m exact_attention_49_amd.build")
            lib = ctypes.CDLL(path)
            for name, (res, args) in EXPORTED_SYMBOLS.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _LIB = lib
    return _LIB


def _check(status: int, what: str) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.attn_status_string(status).decode()
        if status == 6:
            msg += f" (hipError_t {lib.attn_last_hip_error()})"
        raise AttnError(f"{what}: {msg}", status)


def _device_tensor(x: torch.Tensor, name: str) -> None:
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise AttnError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not x.is_contiguous():
        raise AttnError(f"{name} must be contiguous")


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _out_lse(q, out, lse, return_lse, lse_shape, lse_text):
    if out is None:
        out = torch.empty_like(q)
    _device_tensor(out, "out")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise AttnError("out must match q in shape and dtype")
    if lse is None and return_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    if lse is not None:
        _device_tensor(lse, "lse")
        if tuple(lse.shape) != tuple(lse_shape) or lse.dtype != torch.float32:
            raise AttnError(f"lse must be float32 {lse_text}")
    return out, lse


def _check_dtypes(q, k, v):
    if q.dtype not in DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise AttnError("q, k, v must share one dtype: float16 or bfloat16")


def _dense_args(q, k, v, softmax_scale, out, lse, return_lse, grouped):
    """Checks a dense call; k, v may have fewer heads than q when `grouped`."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise AttnError("q must be [B, H, N, d] and k, v [B, Hkv, N, d] with equal shapes")
    bsz, nh, n, d = q.shape
    hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (bsz, n, d):
        raise AttnError("k, v must match q in batch, sequence length and head dim")
    if not grouped and hkv != nh:
        raise AttnError("k, v must have as many heads as q (attn_fwd_gqa takes fewer)")
    _check_dtypes(q, k, v)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    out, lse = _out_lse(q, out, lse, return_lse, (bsz, nh, n), "[B, H, N]")
    return bsz, nh, hkv, n, d, float(softmax_scale), out, lse


def _varlen_args(q, k, v, cu_seqlens, softmax_scale, out, lse, return_lse, grouped):
    """Checks a packed call; k, v may have fewer heads than q when `grouped`."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (cu_seqlens, "cu_seqlens")):
        _device_tensor(t, n)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise AttnError("q must be [H, total_tokens, d] and k, v [Hkv, total_tokens, d]")
    nh, total, d = q.shape
    hkv = k.shape[0]
    if (k.shape[1], k.shape[2]) != (total, d):
        raise AttnError("k, v must match q in total tokens and head dim")
    if not grouped and hkv != nh:
        raise AttnError("k, v must have as many heads as q (attn_fwd_varlen_gqa takes fewer)")
    _check_dtypes(q, k, v)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise AttnError("cu_seqlens must be a 1-D int32 tensor of num_seqs + 1 entries")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    out, lse = _out_lse(q, out, lse, return_lse, (nh, total), "[H, total_tokens]")
    return nh, hkv, total, d, float(softmax_scale), out, lse


def _workspace(nbytes: int, workspace, device):
    """A device workspace of at least nbytes (allocated here, by torch, when none is given)."""
    if nbytes == 0:
        return workspace
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    _device_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise AttnError(f"workspace must hold at least {nbytes} bytes")
    return workspace


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
             window_left: int = -1, window_right: int = -1,
             softmax_scale: float | None = None, out: torch.Tensor | None = None,
             lse: torch.Tensor | None = None, return_lse: bool = True):
    """Dense attention forward.  q, k, v: [B, H, N, d] fp16/bf16 on one GPU.

    Returns (o, lse) with o like q and lse fp32 [B, H, N] (lse is None if return_lse is False
    and no lse buffer was given).  Launches on the current stream."""
    bsz, nh, _, n, d, scale, out, lse = _dense_args(q, k, v, softmax_scale, out, lse,
                                                    return_lse, grouped=False)
    lib = load_library()
    st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      lse.data_ptr() if lse is not None else None, bsz, nh, n, d,
                      DTYPE_CODES[q.dtype], scale, int(bool(causal)),
                      int(window_left), int(window_right), _stream_handle(q.device))
    _check(st, "attn_fwd")
    return out, lse


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = False,
                    window_left: int = -1, window_right: int = -1,
                    softmax_scale: float | None = None, out: torch.Tensor | None = None,
                    lse: torch.Tensor | None = None, return_lse: bool = True):
    """Packed variable-length forward.  q, k, v: [H, total, d]; cu_seqlens: int32 GPU tensor
    [num_seqs + 1]; max_seqlen: a host bound on the sequence lengths.
    Returns (o [H, total, d], lse fp32 [H, total])."""
    nh, _, total, d, scale, out, lse = _varlen_args(q, k, v, cu_seqlens, softmax_scale, out,
                                                    lse, return_lse, grouped=False)
    lib = load_library()
    st = lib.attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None,
                             cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen),
                             total, nh, d, DTYPE_CODES[q.dtype], scale,
                             int(bool(causal)), int(window_left), int(window_right),
                             _stream_handle(q.device))
    _check(st, "attn_fwd_varlen")
    return out, lse


def attn_fwd_gqa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                 window_left: int = -1, window_right: int = -1,
                 softmax_scale: float | None = None, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, return_lse: bool = True):
    """Grouped-query dense forward: q [B, Hq, N, d], k and v [B, Hkv, N, d] with Hkv dividing
    Hq; query head h uses key/value head h // (Hq // Hkv).  Returns (o like q, lse fp32
    [B, Hq, N])."""
    bsz, hq, hkv, n, d, scale, out, lse = _dense_args(q, k, v, softmax_scale, out, lse,
                                                      return_lse, grouped=True)
    lib = load_library()
    st = lib.attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr() if lse is not None else None, bsz, hq, hkv, n, d,
                          DTYPE_CODES[q.dtype], scale, int(bool(causal)),
                          int(window_left), int(window_right), _stream_handle(q.device))
    _check(st, "attn_fwd_gqa")
    return out, lse


def attn_fwd_varlen_gqa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = False,
                        window_left: int = -1, window_right: int = -1,
                        softmax_scale: float | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None, return_lse: bool = True):
    """Grouped-query packed forward: q [Hq, total, d], k and v [Hkv, total, d]."""
    hq, hkv, total, d, scale, out, lse = _varlen_args(q, k, v, cu_seqlens, softmax_scale, out,
                                                      lse, return_lse, grouped=True)
    lib = load_library()
    st = lib.attn_fwd_varlen_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None,
                                 cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen),
                                 total, hq, hkv, d, DTYPE_CODES[q.dtype], scale,
                                 int(bool(causal)), int(window_left), int(window_right),
                                 _stream_handle(q.device))
    _check(st, "attn_fwd_varlen_gqa")
    return out, lse


def attn_fwd_persistent(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                        window_left: int = -1, window_right: int = -1,
                        softmax_scale: float | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None, return_lse: bool = True):
    """attn_fwd_gqa on the persistent schedule (head dim 128): q [B, Hq, N, 128], k and v
    [B, Hkv, N, 128] with Hkv dividing Hq.  Returns (o like q, lse fp32 [B, Hq, N])."""
    bsz, hq, hkv, n, d, scale, out, lse = _dense_args(q, k, v, softmax_scale, out, lse,
                                                      return_lse, grouped=True)
    lib = load_library()
    st = lib.attn_fwd_persistent(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None, bsz, hq, hkv, n,
                                 d, DTYPE_CODES[q.dtype], scale, int(bool(causal)),
                                 int(window_left), int(window_right), _stream_handle(q.device))
    _check(st, "attn_fwd_persistent")
    return out, lse


def attn_fwd_varlen_persistent(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = False,
                               window_left: int = -1, window_right: int = -1,
                               softmax_scale: float | None = None,
                               out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                               return_lse: bool = True):
    """attn_fwd_varlen_gqa on the persistent schedule (head dim 128): q [Hq, total, 128],
    k and v [Hkv, total, 128]."""
    hq, hkv, total, d, scale, out, lse = _varlen_args(q, k, v, cu_seqlens, softmax_scale, out,
                                                      lse, return_lse, grouped=True)
    lib = load_library()
    st = lib.attn_fwd_varlen_persistent(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        out.data_ptr(),
                                        lse.data_ptr() if lse is not None else None,
                                        cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                        int(max_seqlen), total, hq, hkv, d,
                                        DTYPE_CODES[q.dtype], scale, int(bool(causal)),
                                        int(window_left), int(window_right),
                                        _stream_handle(q.device))
    _check(st, "attn_fwd_varlen_persistent")
    return out, lse


def splitkv_num_splits(batch: int, heads: int, seqlen: int, head_dim: int,
                       causal: bool = False, window_left: int = -1) -> int:
    """The split count the library picks for num_splits = 0 (1 = no split)."""
    return load_library().attn_fwd_splitkv_num_splits(batch, heads, seqlen, head_dim,
                                                      int(bool(causal)), int(window_left))


def bwd_workspace_size(batch: int, heads_q: int, seqlen: int) -> int:
    """Workspace bytes attn_bwd needs."""
    return load_library().attn_bwd_workspace_size(batch, heads_q, seqlen)


def varlen_bwd_workspace_size(total_tokens: int, heads_q: int) -> int:
    """Workspace bytes attn_bwd_varlen needs."""
    return load_library().attn_bwd_varlen_workspace_size(total_tokens, heads_q)


def splitkv_workspace_size(batch: int, heads: int, seqlen: int, head_dim: int,
                           num_splits: int = 0, causal: bool = False,
                           window_left: int = -1) -> int:
    """Workspace bytes attn_fwd_splitkv needs (0: none); the mask arguments matter for
    num_splits = 0 only."""
    return load_library().attn_fwd_splitkv_workspace_size(batch, heads, seqlen, head_dim,
                                                          num_splits, int(bool(causal)),
                                                          int(window_left))


def varlen_splitkv_num_splits(num_seqs: int, max_seqlen: int, total_tokens: int, heads: int,
                              head_dim: int) -> int:
    return load_library().attn_fwd_varlen_splitkv_num_splits(num_seqs, max_seqlen,
                                                             total_tokens, heads, head_dim)


def varlen_splitkv_workspace_size(num_seqs: int, max_seqlen: int, total_tokens: int,
                                  heads: int, head_dim: int, num_splits: int = 0) -> int:
    return load_library().attn_fwd_varlen_splitkv_workspace_size(
        num_seqs, max_seqlen, total_tokens, heads, head_dim, num_splits)


def attn_fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                     window_left: int = -1, window_right: int = -1,
                     softmax_scale: float | None = None, out: torch.Tensor | None = None,
                     lse: torch.Tensor | None = None, return_lse: bool = True,
                     num_splits: int = 0, workspace: torch.Tensor | None = None):
    """attn_fwd (or attn_fwd_gqa, when k and v have fewer heads than q) with the key range of
    every q-tile split over num_splits work items (0: the library chooses) and merged.  The
    workspace is allocated here unless one is given."""
    bsz, nh, hkv, n, d, scale, out, lse = _dense_args(q, k, v, softmax_scale, out, lse,
                                                      return_lse, grouped=True)
    lib = load_library()
    nbytes = lib.attn_fwd_splitkv_workspace_size(bsz, nh, n, d, int(num_splits),
                                                 int(bool(causal)), int(window_left))
    ws = _workspace(nbytes, workspace, q.device)
    st = lib.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr() if lse is not None else None, bsz, nh, hkv, n, d,
                              DTYPE_CODES[q.dtype], scale, int(bool(causal)),
                              int(window_left), int(window_right), int(num_splits),
                              ws.data_ptr() if ws is not None else None,
                              ws.numel() * ws.element_size() if ws is not None else 0,
                              _stream_handle(q.device))
    _check(st, "attn_fwd_splitkv")
    return out, lse


def attn_fwd_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             causal: bool = False, window_left: int = -1,
                             window_right: int = -1, softmax_scale: float | None = None,
                             out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                             return_lse: bool = True, num_splits: int = 0):
    """attn_fwd_splitkv with the split partials in the library's static per-GPU scratch
    (ATTN_NOALLOC_SCRATCH_BYTES) instead of a workspace.  The library call allocates nothing;
    pass `out` (and `lse`, or return_lse=False) to keep this wrapper from allocating too."""
    bsz, nh, hkv, n, d, scale, out, lse = _dense_args(q, k, v, softmax_scale, out, lse,
                                                      return_lse, grouped=True)
    lib = load_library()
    st = lib.attn_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr() if lse is not None else None, bsz, nh, hkv,
                                      n, d, DTYPE_CODES[q.dtype], scale, int(bool(causal)),
                                      int(window_left), int(window_right), int(num_splits),
                                      _stream_handle(q.device))
    _check(st, "attn_fwd_splitkv_noalloc")
    return out, lse


def attn_fwd_varlen_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = False,
                            window_left: int = -1, window_right: int = -1,
                            softmax_scale: float | None = None,
                            out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                            return_lse: bool = True, num_splits: int = 0,
                            workspace: torch.Tensor | None = None):
    """attn_fwd_varlen (or attn_fwd_varlen_gqa) with split-KV (see attn_fwd_splitkv)."""
    nh, hkv, total, d, scale, out, lse = _varlen_args(q, k, v, cu_seqlens, softmax_scale, out,
                                                      lse, return_lse, grouped=True)
    lib = load_library()
    ns = cu_seqlens.numel() - 1
    nbytes = lib.attn_fwd_varlen_splitkv_workspace_size(ns, int(max_seqlen), total, nh, d,
                                                        int(num_splits))
    ws = _workspace(nbytes, workspace, q.device)
    st = lib.attn_fwd_varlen_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     cu_seqlens.data_ptr(), ns, int(max_seqlen), total, nh,
                                     hkv, d, DTYPE_CODES[q.dtype], scale, int(bool(causal)),
                                     int(window_left), int(window_right), int(num_splits),
                                     ws.data_ptr() if ws is not None else None,
                                     ws.numel() * ws.element_size() if ws is not None else 0,
                                     _stream_handle(q.device))
    _check(st, "attn_fwd_varlen_splitkv")
    return out, lse


def _grad_outputs(q, k, v, dq, dk, dv):
    out = []
    for g, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if g is None:
            g = torch.empty_like(like)
        _device_tensor(g, name)
        if g.shape != like.shape or g.dtype != like.dtype:
            raise AttnError(f"{name} must match its input in shape and dtype")
        out.append(g)
    return out


def _check_like(x, ref, name, dtype=None):
    _device_tensor(x, name)
    if x.shape != ref.shape or x.dtype != (dtype or ref.dtype):
        raise AttnError(f"{name} has the wrong shape or dtype")


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             lse: torch.Tensor, dout: torch.Tensor, causal: bool = False,
             window_left: int = -1, window_right: int = -1,
             softmax_scale: float | None = None, dq: torch.Tensor | None = None,
             dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None):
    """Backward of attn_fwd / attn_fwd_gqa: q, o, dout [B, Hq, N, d]; k, v [B, Hkv, N, d];
    lse fp32 [B, Hq, N] (the forward's).  Returns (dq, dk, dv), allocated here unless given.
    head_dim 64 or 128.  Launches on the current stream."""
    bsz, hq, hkv, n, d, scale, o, lse = _dense_args(q, k, v, softmax_scale, o, lse, True,
                                                    grouped=True)
    _check_like(dout, q, "dout")
    dq, dk, dv = _grad_outputs(q, k, v, dq, dk, dv)
    lib = load_library()
    ws = _workspace(lib.attn_bwd_workspace_size(bsz, hq, n), workspace, q.device)
    st = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), bsz, hq, hkv,
                      n, d, DTYPE_CODES[q.dtype], scale, int(bool(causal)), int(window_left),
                      int(window_right), ws.data_ptr() if ws is not None else None,
                      ws.numel() * ws.element_size() if ws is not None else 0,
                      _stream_handle(q.device))
    _check(st, "attn_bwd")
    return dq, dk, dv


def attn_bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                    lse: torch.Tensor, dout: torch.Tensor, cu_seqlens: torch.Tensor,
                    max_seqlen: int, causal: bool = False, window_left: int = -1,
                    window_right: int = -1, softmax_scale: float | None = None,
                    dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                    dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Backward of the packed forward: q, o, dout [Hq, total, d]; k, v [Hkv, total, d]; lse fp32
    [Hq, total].  Returns (dq, dk, dv)."""
    hq, hkv, total, d, scale, o, lse = _varlen_args(q, k, v, cu_seqlens, softmax_scale, o, lse,
                                                    True, grouped=True)
    _check_like(dout, q, "dout")
    dq, dk, dv = _grad_outputs(q, k, v, dq, dk, dv)
    lib = load_library()
    ws = _workspace(lib.attn_bwd_varlen_workspace_size(total, hq), workspace, q.device)
    st = lib.attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                             int(max_seqlen), total, hq, hkv, d, DTYPE_CODES[q.dtype], scale,
                             int(bool(causal)), int(window_left), int(window_right),
                             ws.data_ptr() if ws is not None else None,
                             ws.numel() * ws.element_size() if ws is not None else 0,
                             _stream_handle(q.device))
    _check(st, "attn_bwd_varlen")
    return dq, dk, dv


FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)   # E4M3 codes (uint8: the raw bytes)


def _fp8_inputs(q, k, v, dims):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _device_tensor(t, n)
        if t.dtype not in FP8_DTYPES:
            raise AttnError(f"{n} must hold E4M3 codes (torch.float8_e4m3fn or uint8)")
    if q.dim() != dims or k.dim() != dims or v.shape != k.shape:
        raise AttnError("q and k, v have the wrong number of dimensions or k, v differ")


def _descales(descale_q, descale_k, descale_v):
    out = []
    for t, n in ((descale_q, "descale_q"), (descale_k, "descale_k"), (descale_v, "descale_v")):
        if t is None:
            out.append(None)
            continue
        _device_tensor(t, n)
        if t.dtype != torch.float32 or t.numel() != 1:
            raise AttnError(f"{n} must be a one-element float32 GPU tensor")
        out.append(t.data_ptr())
    return out


def _fp8_out(q, out, lse, lse_shape, out_dtype, return_lse):
    if out_dtype not in DTYPE_CODES:
        raise AttnError("out_dtype must be torch.bfloat16 or torch.float16")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _device_tensor(out, "out")
    if out.shape != q.shape or out.dtype != out_dtype:
        raise AttnError("out must have q's shape and out_dtype")
    if lse is None and return_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_like(lse, torch.empty(lse_shape, device="meta"), "lse", torch.float32)
    return out, lse


def attn_fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 descale_q: torch.Tensor | None = None, descale_k: torch.Tensor | None = None,
                 descale_v: torch.Tensor | None = None, causal: bool = False,
                 window_left: int = -1, window_right: int = -1,
                 softmax_scale: float | None = None, out_dtype: torch.dtype = torch.bfloat16,
                 out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                 return_lse: bool = True):
    """FP8 forward: q [B, Hq, N, d], k, v [B, Hkv, N, d] as E4M3 codes (d = 64, 128 or 256);
    descales are one-element fp32 GPU tensors or None (= 1).  Returns (o in out_dtype, lse
    fp32)."""
    _fp8_inputs(q, k, v, 4)
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (bsz, n, d):
        raise AttnError("k, v must match q in batch, sequence length and head dim")
    scale = float(softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d))
    dq, dk, dv = _descales(descale_q, descale_k, descale_v)
    out, lse = _fp8_out(q, out, lse, (bsz, hq, n), out_dtype, return_lse)
    lib = load_library()
    st = lib.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr() if lse is not None else None, dq, dk, dv, bsz, hq,
                          hkv, n, d, DTYPE_CODES[out_dtype], scale, int(bool(causal)),
                          int(window_left), int(window_right), _stream_handle(q.device))
    _check(st, "attn_fwd_fp8")
    return out, lse


def attn_fwd_varlen_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        cu_seqlens: torch.Tensor, max_seqlen: int,
                        descale_q: torch.Tensor | None = None,
                        descale_k: torch.Tensor | None = None,
                        descale_v: torch.Tensor | None = None, causal: bool = False,
                        window_left: int = -1, window_right: int = -1,
                        softmax_scale: float | None = None,
                        out_dtype: torch.dtype = torch.bfloat16,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        return_lse: bool = True):
    """Packed FP8 forward: q [Hq, total, d], k, v [Hkv, total, d] E4M3 codes."""
    _fp8_inputs(q, k, v, 3)
    _device_tensor(cu_seqlens, "cu_seqlens")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise AttnError("cu_seqlens must be a 1-D int32 tensor of num_seqs + 1 entries")
    hq, total, d = q.shape
    hkv = k.shape[0]
    if (k.shape[1], k.shape[2]) != (total, d):
        raise AttnError("k, v must match q in total tokens and head dim")
    scale = float(softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d))
    dq, dk, dv = _descales(descale_q, descale_k, descale_v)
    out, lse = _fp8_out(q, out, lse, (hq, total), out_dtype, return_lse)
    lib = load_library()
    st = lib.attn_fwd_varlen_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None, dq, dk, dv,
                                 cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(max_seqlen),
                                 total, hq, hkv, d, DTYPE_CODES[out_dtype], scale,
                                 int(bool(causal)), int(window_left), int(window_right),
                                 _stream_handle(q.device))
    _check(st, "attn_fwd_varlen_fp8")
    return out, lse


def device_info(device: int = 0) -> dict:
    """Compute units and peak engine clock (MHz) of a HIP device, from the HIP runtime."""
    lib = load_library()
    cus, clk = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib.attn_device_info(int(device), ctypes.byref(cus), ctypes.byref(clk)),
           "attn_device_info")
    return {"compute_units": cus.value, "clock_mhz": clk.value / 1000.0}
