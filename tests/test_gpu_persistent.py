"""GPU parity of the persistent ping-pong kernel (attn_fwd_persistent, attn_fwd_varlen_persistent;
head dim 128): one workgroup per compute unit sweeps a list of q-tiles as one pipeline.  The cases stress the list: many q-tiles
per workgroup, packed batches whose q-tiles have a single key tile (the tile loads then look
further down the list), empty and one-token sequences (slots with nothing to compute), masks,
and grouped K/V heads.  Every compared head is compared in full with the fp64 oracle.  The
grouped-head packing of the default grid-launched ping-pong kernel is checked here too."""

import math

import pytest
import torch

import bench
from exact_attention_49_amd import (AttnError, attn_fwd, attn_fwd_gqa, attn_fwd_persistent,
                                    attn_fwd_varlen_persistent, inputs)
from tests.gpu_helpers import check_all_heads_dense, check_all_heads_varlen

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
    o, lse = attn_fwd_varlen_persistent(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV),
                                        max(SHORT_MIX), causal=causal, window_left=wl,
                                        window_right=wr)
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
    o, lse = attn_fwd_persistent(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    sel = sorted({0, h // 2, h - 1})
    for hd in sel:
        sl = slice(hd, hd + 1)
        check_all_heads_dense(q[:, sl], k[:, sl], v[:, sl], o[:, sl], lse[:, sl],
                              1 / math.sqrt(128), causal, -1, -1, DTYPES[dt], f"head {hd}")


# (B, Hq, Hkv, N): grouped K/V heads on the ping-pong kernels; the query heads of a K/V head
# are packed into one q-tile by the largest power of two dividing the group, at most 8:
# MQA (group 32: 8 heads of 32 positions per q-tile), group 3 (no packing), group 6 (2 heads
# of 128 positions), group 12 (4 heads of 64 positions, ragged N)
PACKED = [(1, 32, 1, 4096), (1, 36, 12, 4096), (1, 48, 8, 2048), (2, 24, 2, 2100)]
PACK_MASKS = {"none": (False, -1, -1), "causal": (True, -1, -1), "window_30_70": (False, 30, 70),
              "causal_w200": (True, 200, -1)}


@pytest.mark.parametrize("mask", list(PACK_MASKS))
@pytest.mark.parametrize("shape", PACKED)
def test_packed_heads_match_repeated_kv_and_oracle(shape, mask):
    """A packed q-tile computes each of its heads' rows with the same key tiles, in the same
    order, as an unpacked one: the grouped call must equal attn_fwd on K/V repeated along the
    heads bit for bit, and match the oracle (first, middle and last query head in full)."""
    b, hq, hkv, n = shape
    causal, wl, wr = PACK_MASKS[mask]
    print(f"[case] packed heads {shape} {mask}", flush=True)
    q, k, v = inputs.make_dense(b, hq, n, 128, "bf16", seed=1700 + hq + hkv, heads_kv=hkv)
    w = inputs.Workload(name="t", heads=hq, heads_kv=hkv, head_dim=128, dtype="bf16",
                        causal=causal, seed=0, batch=b, seqlen=n, window_left=wl,
                        window_right=wr)
    assert bench.kernel_name(w) == "attn_fwd_pp_kernel"
    o, lse = attn_fwd_gqa(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_left=wl,
                          window_right=wr)
    g = hq // hkv
    o2, lse2 = attn_fwd(q.to(DEV), k.repeat_interleave(g, 1).to(DEV),
                        v.repeat_interleave(g, 1).to(DEV), causal=causal, window_left=wl,
                        window_right=wr)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for hd in sorted({0, hq // 2, hq - 1}):
        sl = slice(hd, hd + 1)
        kh = slice(hd // g, hd // g + 1)
        check_all_heads_dense(q[:, sl], k[:, kh], v[:, kh], o[:, sl], lse[:, sl],
                              1 / math.sqrt(128), causal, wl, wr, torch.bfloat16, f"head {hd}")


@pytest.mark.parametrize("mask", ["none", "causal", "causal_w200"])
@pytest.mark.parametrize("shape", PACKED)
def test_persistent_packed_heads_match_oracle(shape, mask):
    """The persistent kernel on grouped K/V heads (packed q-tiles): first, middle and last
    query head in full against the oracle."""
    b, hq, hkv, n = shape
    causal, wl, wr = PACK_MASKS[mask]
    print(f"[case] persistent packed heads {shape} {mask}", flush=True)
    q, k, v = inputs.make_dense(b, hq, n, 128, "bf16", seed=1800 + hq + hkv, heads_kv=hkv)
    o, lse = attn_fwd_persistent(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal,
                                 window_left=wl, window_right=wr)
    torch.cuda.synchronize()
    g = hq // hkv
    for hd in sorted({0, hq // 2, hq - 1}):
        sl = slice(hd, hd + 1)
        kh = slice(hd // g, hd // g + 1)
        check_all_heads_dense(q[:, sl], k[:, kh], v[:, kh], o[:, sl], lse[:, sl],
                              1 / math.sqrt(128), causal, wl, wr, torch.bfloat16, f"head {hd}")


def test_persistent_rejects_other_head_dims():
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(AttnError, match="UNSUPPORTED_HEAD_DIM"):
        attn_fwd_persistent(q, q, q)


@pytest.mark.parametrize("mask", ["causal", "none", "causal_w200"])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (24, 2)])
def test_packed_heads_varlen_default_path(hq, hkv, mask):
    """Packed query heads on a packed batch through the default entry point (grid-launched
    ping-pong kernel): bitwise equal to attn_fwd_varlen on repeated K/V, and three query heads
    in full against the oracle.  Lengths include empty, one-token and ragged sequences."""
    from exact_attention_49_amd import attn_fwd_varlen, attn_fwd_varlen_gqa
    causal, wl, wr = PACK_MASKS[mask]
    lens = [700, 0, 1, 513, 1290, 64, 257, 900, 3, 400]
    print(f"[case] packed heads varlen default Hq{hq} Hkv{hkv} {mask}", flush=True)
    q, k, v, cu = inputs.make_varlen(len(lens), 0, 0, hq, 128, "bf16", seed=1900 + hq + hkv,
                                     lengths=lens, heads_kv=hkv)
    w = inputs.Workload(name="t", heads=hq, heads_kv=hkv, head_dim=128, dtype="bf16",
                        causal=causal, seed=0, num_seqs=len(lens), window_left=wl,
                        window_right=wr)
    assert bench.kernel_name(w, cu) == "attn_fwd_pp_kernel"
    o, lse = attn_fwd_varlen_gqa(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lens),
                                 causal=causal, window_left=wl, window_right=wr)
    g = hq // hkv
    o2, lse2 = attn_fwd_varlen(q.to(DEV), k.repeat_interleave(g, 0).to(DEV),
                               v.repeat_interleave(g, 0).to(DEV), cu.to(DEV), max(lens),
                               causal=causal, window_left=wl, window_right=wr)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for hd in sorted({0, hq // 2, hq - 1}):
        sl = slice(hd, hd + 1)
        kh = slice(hd // g, hd // g + 1)
        check_all_heads_varlen(q[sl], k[kh], v[kh], cu, o[sl], lse[sl], 1 / math.sqrt(128),
                               causal, wl, wr, torch.bfloat16, f"head {hd}")


@pytest.mark.parametrize("mask", ["causal", "window_30_70"])
def test_packed_heads_fp16(mask):
    """fp16 on the packed ping-pong kernel (group 8: 8 heads of 32 positions per q-tile)."""
    from exact_attention_49_amd import attn_fwd, attn_fwd_gqa
    b, hq, hkv, n = 2, 32, 4, 2100
    causal, wl, wr = PACK_MASKS[mask]
    print(f"[case] packed heads fp16 {mask}", flush=True)
    q, k, v = inputs.make_dense(b, hq, n, 128, "fp16", seed=1950, heads_kv=hkv)
    w = inputs.Workload(name="t", heads=hq, heads_kv=hkv, head_dim=128, dtype="fp16",
                        causal=causal, seed=0, batch=b, seqlen=n, window_left=wl,
                        window_right=wr)
    assert bench.kernel_name(w) == "attn_fwd_pp_kernel"
    o, lse = attn_fwd_gqa(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_left=wl,
                          window_right=wr)
    g = hq // hkv
    o2, lse2 = attn_fwd(q.to(DEV), k.repeat_interleave(g, 1).to(DEV),
                        v.repeat_interleave(g, 1).to(DEV), causal=causal, window_left=wl,
                        window_right=wr)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for hd in (0, hq - 1):
        sl = slice(hd, hd + 1)
        kh = slice(hd // g, hd // g + 1)
        check_all_heads_dense(q[:, sl], k[:, kh], v[:, kh], o[:, sl], lse[:, sl],
                              1 / math.sqrt(128), causal, wl, wr, torch.float16, f"head {hd}")
