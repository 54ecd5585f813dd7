"""GPU parity of the persistent ping-pong kernel (head dim 128, big grids): one workgroup per
compute unit sweeps a list of q-tiles as one pipeline.  The cases stress the list: many q-tiles
per workgroup, packed batches whose q-tiles have a single key tile (the tile loads then look
further down the list), empty and one-token sequences (slots with nothing to compute), masks,
and grouped K/V heads.  Every compared head is compared in full with the fp64 oracle."""

import math

import pytest
import torch

import bench
from exact_attention_49_amd import attn_fwd_varlen_gqa, inputs
from tests.gpu_helpers import check_all_heads_dense, check_all_heads_varlen, gpu_dense

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}

# lengths with q-tiles of one key tile (<= 64 rows, unmasked), empty and one-token sequences
SHORT_MIX = [1, 64, 0, 65, 300, 700, 3, 256, 257, 40]


@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (True, -1, -1), (False, 30, 70),
                                          (True, 100, -1)])
@pytest.mark.parametrize("hkv", [96, 24])
def test_persistent_packed_short_sequences(causal, wl, wr, hkv):
    print(f"[case] persistent packed causal={causal} wl={wl} wr={wr} hkv={hkv}", flush=True)
    heads = 96   # 96 heads x 12 q-tiles of 256 rows: 1152 slots, about 4.5 per workgroup
    q, k, v, cu = inputs.make_varlen(len(SHORT_MIX), 0, 0, heads, 128, "bf16", seed=1500 + hkv,
                                     lengths=SHORT_MIX, heads_kv=hkv)
    w = inputs.Workload(name="t", heads=heads, head_dim=128, dtype="bf16", causal=causal,
                        seed=0, num_seqs=len(SHORT_MIX), window_left=wl, window_right=wr)
    assert bench.kernel_name(w, cu) == "attn_fwd_pp_kernel"
    o, lse = attn_fwd_varlen_gqa(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(SHORT_MIX),
                                 causal=causal, window_left=wl, window_right=wr)
    torch.cuda.synchronize()
    check_all_heads_varlen(q, k, v, cu, o, lse, 1 / math.sqrt(128), causal, wl, wr,
                           torch.bfloat16, "persistent packed")


@pytest.mark.parametrize("shape,causal,dt", [((1, 1024, 768), False, "fp16"),
                                             ((3, 200, 1100), True, "bf16"),
                                             ((1, 300, 64), False, "bf16")])
def test_persistent_dense_many_items(shape, causal, dt):
    """B1 H1024 N768: 3072 slots, 12 q-tiles per workgroup; B3 H200 N1100 causal: 5 q-tiles
    per head with a ragged last one; B1 H300 N64: 300 q-tiles of a single key tile each (the
    loads run two q-tiles ahead).  A head from each end and the middle, in full."""
    b, h, n = shape
    print(f"[case] persistent dense B{b} H{h} N{n} causal={causal} {dt}", flush=True)
    q, k, v = inputs.make_dense(b, h, n, 128, dt, seed=1600 + h)
    o, lse = gpu_dense(q, k, v, causal)
    sel = sorted({0, h // 2, h - 1})
    for hd in sel:
        sl = slice(hd, hd + 1)
        check_all_heads_dense(q[:, sl], k[:, sl], v[:, sl], o[:, sl], lse[:, sl],
                              1 / math.sqrt(128), causal, -1, -1, DTYPES[dt], f"head {hd}")
