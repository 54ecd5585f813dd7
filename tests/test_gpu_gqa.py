"""GPU parity of the grouped-query entry points (through the C ABI) against the fp64 CPU
oracle, which gives query head h the key/value head h // (Hq / Hkv).

Cases: every head dim, both dtypes, the mask modes, GQA and MQA (one key/value head), packed
batches, split-KV with grouped heads, grids large enough for the big-tile kernels, and the
grouped workload at full size on sampled rows.  On every kernel, a grouped call must also be
bit-identical to the plain call on K and V repeated along the head axis: each query head's
arithmetic is the same, only the address of its K/V head differs."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_49_amd import (attn_fwd, attn_fwd_gqa, attn_fwd_splitkv,
                                    attn_fwd_varlen, attn_fwd_varlen_gqa,
                                    attn_fwd_varlen_splitkv, inputs)
from tests.gpu_helpers import assert_close, check_all_heads_dense, sample_rows, to64

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
MASKS = {
    "none": dict(causal=False, wl=-1, wr=-1),
    "causal": dict(causal=True, wl=-1, wr=-1),
    "window_40_0": dict(causal=True, wl=40, wr=0),
    "window_30_70": dict(causal=False, wl=30, wr=70),
}
DEV = torch.device("cuda:0")


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _gqa(q, k, v, m):
    o, lse = attn_fwd_gqa(q.to(DEV), k.to(DEV), v.to(DEV), causal=m["causal"],
                          window_left=m["wl"], window_right=m["wr"])
    torch.cuda.synchronize()
    return o, lse


def _at(x, idx):
    """Entries of x at the (b, h, row) triples of idx, as float64 numpy."""
    t = torch.from_numpy(idx).to(x.device)
    return to64(x[t[:, 0], t[:, 1], t[:, 2]])


def _oracle(q, k, v, scale, m):
    return oracle.attention_dense(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                  scale, m["causal"], m["wl"], m["wr"])


@pytest.mark.parametrize("hq,hkv", [(4, 2), (6, 1)])
@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("dtype", list(DTYPES))
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_gqa_dense_all_modes(d, dtype, mask, hq, hkv):
    _announce(f"gqa dense d={d} {dtype} {mask} hq={hq} hkv={hkv}")
    q, k, v = inputs.make_dense(2, hq, 203, d, dtype, seed=1000 + d + hq, heads_kv=hkv)
    o, lse = _gqa(q, k, v, MASKS[mask])
    o_ref, lse_ref = _oracle(q, k, v, 1 / math.sqrt(d), MASKS[mask])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, DTYPES[dtype],
                 f"gqa d={d} {dtype} {mask} {hq}/{hkv}")


# (B, Hq, Hkv, N, d): shapes whose grids reach each kernel family, big tiles included
BIG_SHAPES = [(1, 32, 8, 4096, 128), (2, 16, 1, 2048, 128), (1, 32, 4, 1500, 64),
              (1, 8, 2, 1100, 256), (1, 4, 1, 700, 512)]


@pytest.mark.parametrize("shape", BIG_SHAPES)
@pytest.mark.parametrize("mask", ["causal", "window_40_0", "none"])
def test_gqa_is_bitwise_mha_on_repeated_kv(shape, mask):
    bsz, hq, hkv, n, d = shape
    _announce(f"gqa == mha(repeat) {shape} {mask}")
    m = MASKS[mask]
    q, k, v = inputs.make_dense(bsz, hq, n, d, "bf16", seed=1100 + n + d, heads_kv=hkv)
    o, lse = _gqa(q, k, v, m)
    g = hq // hkv
    kr = k.repeat_interleave(g, dim=1).contiguous()
    vr = v.repeat_interleave(g, dim=1).contiguous()
    o2, lse2 = attn_fwd(q.to(DEV), kr.to(DEV), vr.to(DEV), causal=m["causal"],
                        window_left=m["wl"], window_right=m["wr"])
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), o2.cpu())
    assert torch.equal(lse.cpu(), lse2.cpu())
    # and sampled rows of a few heads against the oracle
    rng = np.random.default_rng(n)
    idx = np.array([(b, h, r) for b in range(bsz) for h in (0, hq - 1, hq // 2)
                    for r in sample_rows(n, rng, extra=3)])
    o_ref, lse_ref = oracle.attention_rows_dense(q.float().numpy(), k.float().numpy(),
                                                 v.float().numpy(), idx, 1 / math.sqrt(d),
                                                 m["causal"], m["wl"], m["wr"])
    assert_close(_at(o, idx), _at(lse, idx), o_ref, lse_ref, torch.bfloat16, f"{shape} {mask}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mask", ["causal", "window_30_70"])
def test_gqa_varlen(d, mask):
    _announce(f"gqa varlen d={d} {mask}")
    m = MASKS[mask]
    lens = [1, 0, 64, 300, 777, 129, 3]
    q, k, v, cu = inputs.make_varlen(len(lens), 0, 0, 6, d, "fp16", seed=1200 + d,
                                     lengths=lens, heads_kv=2)
    o, lse = attn_fwd_varlen_gqa(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lens),
                                 causal=m["causal"], window_left=m["wl"], window_right=m["wr"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen(q.float().numpy(), k.float().numpy(),
                                             v.float().numpy(), cu.numpy(), 1 / math.sqrt(d),
                                             m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.float16, f"varlen d={d} {mask}")
    # the packed grouped call equals the packed plain call on repeated K/V, bit for bit
    o2, lse2 = attn_fwd_varlen(q.to(DEV), k.repeat_interleave(3, 0).to(DEV),
                               v.repeat_interleave(3, 0).to(DEV), cu.to(DEV), max(lens),
                               causal=m["causal"], window_left=m["wl"], window_right=m["wr"])
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), o2.cpu()) and torch.equal(lse.cpu(), lse2.cpu())


@pytest.mark.parametrize("d", [64, 128, 512])
def test_gqa_splitkv(d):
    _announce(f"gqa split-KV d={d}")
    m = MASKS["causal"]
    # 8 query heads (work dealt to the XCDs in contiguous ranges) and 3 (dealt item by item)
    for hq, hkv in ((8, 2), (3, 1)):
        q, k, v = inputs.make_dense(1, hq, 900, d, "bf16", seed=1300 + d + hq, heads_kv=hkv)
        o, lse = attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, num_splits=5)
        torch.cuda.synchronize()
        o_ref, lse_ref = _oracle(q, k, v, 1 / math.sqrt(d), m)
        assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16,
                     f"split d={d} Hq{hq} Hkv{hkv}")
    lens = [300, 0, 600]
    q, k, v, cu = inputs.make_varlen(3, 0, 0, 4, d, "bf16", seed=1350 + d, lengths=lens,
                                     heads_kv=1)
    o, lse = attn_fwd_varlen_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), 600,
                                     causal=True, window_left=200, window_right=0,
                                     num_splits=3)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen(q.float().numpy(), k.float().numpy(),
                                             v.float().numpy(), cu.numpy(), 1 / math.sqrt(d),
                                             True, 200, 0)
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"split varlen d={d}")


def test_gqa_binding_rejects_non_divisor_heads():
    q = torch.zeros(1, 6, 16, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16, device=DEV)
    from exact_attention_49_amd import AttnError
    with pytest.raises(AttnError):
        attn_fwd_gqa(q, k, k)
    with pytest.raises(AttnError):
        attn_fwd(q, k, k)   # the plain call wants equal head counts


def test_workload_gqa_bf16_d128_hq32_hkv8_n8192_full():
    """The grouped-query workload (packed q-tiles on the ping-pong kernel): every row of every
    query head against the oracle."""
    w = inputs.WORKLOADS["gqa_bf16_d128_hq32_hkv8_n8192"]
    _announce(w.name)
    q, k, v = inputs.make_workload(w)
    m = dict(causal=w.causal, wl=w.window_left, wr=w.window_right)
    o, lse = _gqa(q, k, v, m)
    check_all_heads_dense(q, k, v, o, lse, w.softmax_scale, w.causal, w.window_left,
                          w.window_right, w.torch_dtype, w.name)
