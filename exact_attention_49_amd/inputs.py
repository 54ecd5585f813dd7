"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and names shapes; it holds none of the attention
arithmetic.  Both the HIP path and the CPU oracle consume the tensors it returns, already
rounded to the I/O dtype, so they see identical inputs.

Recipe: a CPU `torch.Generator` seeded with the workload's seed draws, in this order,
(for packed batches) the sequence lengths with `randint`, then Q, K and V with `randn` in
float32 (K and V with the key/value head count, which is below Q's for grouped-query
problems); Q, K and V are multiplied by the workload's value scale (an exact power of two)
and cast to the I/O dtype with round-to-nearest-even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "make_dense", "make_varlen", "make_workload",
           "make_upstream", "quantize_fp8"]

_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One synthetic attention problem.

    Dense workloads use `batch`, `seqlen`; packed workloads draw `num_seqs` lengths uniformly
    from [min_len, max_len] (inclusive).  `window_left`/`window_right` of -1 mean unbounded.
    """

    name: str
    heads: int
    head_dim: int
    dtype: str
    causal: bool
    seed: int
    batch: int = 1
    seqlen: int = 0
    num_seqs: int = 0
    min_len: int = 0
    max_len: int = 0
    window_left: int = -1
    window_right: int = -1
    value_scale: float = 1.0
    heads_kv: int = 0       # key/value heads (grouped-query attention); 0: as many as `heads`
    splitkv: bool = False   # run through the split-KV entry point
    backward: bool = False  # time the backward pass (dO drawn with seed + 100)
    fp8: bool = False       # E4M3 inputs (drawn as `dtype`, then quantize_fp8 per tensor)
    note: str = field(default="", compare=False)

    @property
    def varlen(self) -> bool:
        return self.num_seqs > 0

    @property
    def kv_heads(self) -> int:
        return self.heads_kv or self.heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp16_d64", batch=1, heads=1, seqlen=128, head_dim=64, dtype="fp16",
                 causal=False, seed=4901, note="B=1 H=1 N=128 d=64 fp16 non-causal"),
        Workload("causal_bf16_d128_n2048", batch=4, heads=16, seqlen=2048, head_dim=128,
                 dtype="bf16", causal=True, seed=4902,
                 note="B=4 H=16 N=2048 d=128 bf16 causal, O and LSE"),
        Workload("causal_bf16_d128_n8192", batch=2, heads=32, seqlen=8192, head_dim=128,
                 dtype="bf16", causal=True, seed=4903, value_scale=0.5,
                 note="B=2 H=32 N=8192 d=128 bf16 causal, inputs N(0,1)*0.5"),
        Workload("varlen_bf16_d64_w1024", heads=32, head_dim=64, dtype="bf16", causal=True,
                 seed=4904, num_seqs=16, min_len=64, max_len=4096, window_left=1024,
                 window_right=0,
                 note="16 packed sequences, lengths U[64,4096], H=32 d=64 bf16 causal, "
                      "sliding window 1024 (keys i-1024..i)"),
        Workload("dense_fp16_d512_n4096", batch=1, heads=8, seqlen=4096, head_dim=512,
                 dtype="fp16", causal=False, seed=4905,
                 note="B=1 H=8 N=4096 d=512 fp16 non-causal"),
        # a long problem with few heads: its plain grid (2 x 128 q-tiles) cannot fill the
        # chip, the case split-KV is for
        Workload("splitkv_bf16_d128_h2_n16384", batch=1, heads=2, seqlen=16384,
                 head_dim=128, dtype="bf16", causal=True, seed=4906, splitkv=True,
                 note="B=1 H=2 N=16384 d=128 bf16 causal, split-KV (low occupancy)"),
        # grouped-query attention: 32 query heads on 8 key/value heads (groups of 4)
        Workload("gqa_bf16_d128_hq32_hkv8_n8192", batch=2, heads=32, heads_kv=8,
                 seqlen=8192, head_dim=128, dtype="bf16", causal=True, seed=4907,
                 value_scale=0.5,
                 note="B=2 Hq=32 Hkv=8 N=8192 d=128 bf16 causal, inputs N(0,1)*0.5"),
        # the FP8 forward on the forward benchmark's shape (bf16 output)
        Workload("fp8_causal_d128_n8192", batch=2, heads=32, seqlen=8192, head_dim=128,
                 dtype="bf16", causal=True, seed=4908, fp8=True,
                 note="B=2 H=32 N=8192 d=128 causal, E4M3 Q/K/V with per-tensor descales, "
                      "bf16 O"),
        # the backward pass on the forward benchmark's shape
        Workload("bwd_causal_bf16_d128_n8192", batch=2, heads=32, seqlen=8192, head_dim=128,
                 dtype="bf16", causal=True, seed=4903, value_scale=0.5, backward=True,
                 note="backward of B=2 H=32 N=8192 d=128 bf16 causal (dQ, dK, dV)"),
    ]
}


def _randn_qkv(gen: torch.Generator, shape, kv_shape, dtype: torch.dtype, value_scale: float):
    out = []
    for sh in (shape, kv_shape, kv_shape):
        x = torch.randn(sh, generator=gen, dtype=torch.float32)
        if value_scale != 1.0:
            x = x * value_scale
        out.append(x.to(dtype))
    return out


def make_dense(batch: int, heads: int, seqlen: int, head_dim: int, dtype: str, seed: int,
               value_scale: float = 1.0, heads_kv: int = 0):
    """Q [B, H, N, d] and K, V [B, Hkv, N, d] (Hkv = heads_kv, or H when 0) as contiguous CPU
    tensors in the I/O dtype."""
    gen = torch.Generator("cpu").manual_seed(seed)
    return _randn_qkv(gen, (batch, heads, seqlen, head_dim),
                      (batch, heads_kv or heads, seqlen, head_dim), _DTYPES[dtype], value_scale)


def make_varlen(num_seqs: int, min_len: int, max_len: int, heads: int, head_dim: int,
                dtype: str, seed: int, value_scale: float = 1.0, lengths=None,
                heads_kv: int = 0):
    """Q [H, total, d] and K, V [Hkv, total, d] as contiguous CPU tensors plus int32
    cu_seqlens [num_seqs + 1].

    Lengths are drawn uniformly from [min_len, max_len] unless `lengths` is given."""
    gen = torch.Generator("cpu").manual_seed(seed)
    if lengths is None:
        lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=gen, dtype=torch.int64)
    else:
        lens = torch.as_tensor(list(lengths), dtype=torch.int64)
    cu = torch.zeros(lens.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    total = int(cu[-1])
    q, k, v = _randn_qkv(gen, (heads, total, head_dim), (heads_kv or heads, total, head_dim),
                         _DTYPES[dtype], value_scale)
    return q, k, v, cu.to(torch.int32)


def make_workload(w: Workload):
    """Tensors for a named workload: (q, k, v) dense or (q, k, v, cu_seqlens) packed."""
    if w.varlen:
        return make_varlen(w.num_seqs, w.min_len, w.max_len, w.heads, w.head_dim, w.dtype,
                           w.seed, w.value_scale, heads_kv=w.heads_kv)
    return make_dense(w.batch, w.heads, w.seqlen, w.head_dim, w.dtype, w.seed, w.value_scale,
                      heads_kv=w.heads_kv)


def make_upstream(shape, dtype: str, seed: int, value_scale: float = 1.0):
    """An upstream gradient dO of the given shape: `randn` in float32 from a CPU generator
    seeded with `seed`, times the value scale, cast to the I/O dtype (as Q, K, V)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    if value_scale != 1.0:
        x = x * value_scale
    return x.to(_DTYPES[dtype])


E4M3_MAX = 448.0


def quantize_fp8(x: torch.Tensor):
    """Per-tensor E4M3 quantisation of an input: descale = amax / 448 (as fp32) and codes =
    x / descale cast to torch.float8_e4m3fn (round to nearest even).  Returns (codes,
    descale); the codes stand for codes * descale."""
    x = x.float()
    descale = float(torch.tensor(float(x.abs().max()) / E4M3_MAX, dtype=torch.float32))
    if descale == 0.0:
        descale = 1.0
    return (x / descale).to(torch.float8_e4m3fn), descale
