"""GPU parity: the HIP kernels (through the C ABI) against the fp64 CPU oracle.

Small shapes are compared in full (they span several q-tiles and K/V tiles plus a ragged
tail); the five named workloads are compared in full, every row of every head, in the launch
configuration the benchmark times; plus properties that hold at any size."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_49_amd import AttnError, attn_fwd, attn_fwd_varlen, inputs
from tests.gpu_helpers import (O_TOL, assert_close, check_all_heads_dense,
                               check_all_heads_varlen, gpu_dense, gpu_varlen, oracle_dense, to64)

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
MASKS = {
    "none": dict(causal=False, wl=-1, wr=-1),
    "causal": dict(causal=True, wl=-1, wr=-1),
    "causal_w37": dict(causal=True, wl=37, wr=-1),
    "window_50_20": dict(causal=False, wl=50, wr=20),
    "right_only_5": dict(causal=False, wl=-1, wr=5),
    "left_only_70": dict(causal=False, wl=70, wr=-1),
}


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("dtype", list(DTYPES))
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_dense_small_all_modes(d, dtype, mask):
    _announce(f"dense d={d} {dtype} {mask}")
    m = MASKS[mask]
    q, k, v = inputs.make_dense(2, 2, 300, d, dtype, seed=100 + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu_dense(q, k, v, m["causal"], m["wl"], m["wr"])
    o_ref, lse_ref = oracle_dense(q, k, v, scale, m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, DTYPES[dtype], f"d={d} {dtype} {mask}")


@pytest.mark.parametrize("n", [1, 2, 31, 33, 255, 256, 257, 513])
@pytest.mark.parametrize("mask", ["none", "causal", "causal_w37"])
def test_dense_ragged_lengths(n, mask):
    _announce(f"dense ragged n={n} {mask}")
    m = MASKS[mask]
    q, k, v = inputs.make_dense(1, 3, n, 128, "bf16", seed=200 + n)
    o, lse = gpu_dense(q, k, v, m["causal"], m["wl"], m["wr"])
    o_ref, lse_ref = oracle_dense(q, k, v, 1 / math.sqrt(128), m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"n={n} {mask}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "causal_w37", "window_50_20"])
def test_varlen_small(d, mask):
    _announce(f"varlen small d={d} {mask}")
    m = MASKS[mask]
    lens = [1, 0, 64, 300, 1000, 257, 3]
    q, k, v, cu = inputs.make_varlen(len(lens), 0, 0, 3, d, "bf16", seed=300 + d, lengths=lens)
    o, lse = gpu_varlen(q, k, v, cu, m["causal"], m["wl"], m["wr"])
    o_ref, lse_ref = oracle.attention_varlen(q.float().numpy(), k.float().numpy(),
                                             v.float().numpy(), cu.numpy(), 1 / math.sqrt(d),
                                             m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"varlen d={d} {mask}")


def test_varlen_equals_dense_per_sequence():
    _announce("varlen == dense per sequence")
    lens = [129, 700, 5]
    q, k, v, cu = inputs.make_varlen(3, 0, 0, 2, 128, "fp16", seed=11, lengths=lens)
    o, lse = gpu_varlen(q, k, v, cu, True, 100, -1)
    for s, (a, b) in enumerate(zip(cu[:-1].tolist(), cu[1:].tolist())):
        od, ld = gpu_dense(q[None, :, a:b].contiguous(), k[None, :, a:b].contiguous(),
                           v[None, :, a:b].contiguous(), True, 100, -1)
        assert torch.equal(od[0].cpu(), o[:, a:b].cpu()), s
        assert torch.equal(ld[0].cpu(), lse[:, a:b].cpu()), s


# ---------------------------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------------------------

def _dense_workload(name):
    w = inputs.WORKLOADS[name]
    q, k, v = inputs.make_workload(w)
    return w, q, k, v


def test_workload_tiny_fp16_d64_full():
    w, q, k, v = _dense_workload("tiny_fp16_d64")
    _announce(w.name)
    o, lse = gpu_dense(q, k, v, w.causal, w.window_left, w.window_right)
    o_ref, lse_ref = oracle_dense(q, k, v, w.softmax_scale, w.causal, w.window_left,
                                  w.window_right)
    assert_close(to64(o), to64(lse), o_ref, lse_ref, w.torch_dtype, w.name)


def _check_finite(o, lse):
    assert bool(torch.isfinite(o).all()), "non-finite O"
    assert bool(torch.isfinite(lse).all()), "non-finite LSE"


def test_workload_causal_bf16_d128_n2048_full():
    w, q, k, v = _dense_workload("causal_bf16_d128_n2048")
    _announce(w.name)
    o, lse = gpu_dense(q, k, v, w.causal)
    _check_finite(o, lse)
    check_all_heads_dense(q, k, v, o, lse, w.softmax_scale, w.causal, w.window_left,
                          w.window_right, w.torch_dtype, w.name)


def test_workload_causal_bf16_d128_n8192_full():
    """Every row of all 64 (batch, head) pairs (the benchmark's launch: the persistent
    ping-pong kernel)."""
    w, q, k, v = _dense_workload("causal_bf16_d128_n8192")
    _announce(w.name)
    o, lse = gpu_dense(q, k, v, w.causal)
    _check_finite(o, lse)
    check_all_heads_dense(q, k, v, o, lse, w.softmax_scale, w.causal, w.window_left,
                          w.window_right, w.torch_dtype, w.name)


def test_workload_dense_fp16_d512_n4096_full():
    w, q, k, v = _dense_workload("dense_fp16_d512_n4096")
    _announce(w.name)
    o, lse = gpu_dense(q, k, v, w.causal)
    _check_finite(o, lse)
    check_all_heads_dense(q, k, v, o, lse, w.softmax_scale, w.causal, w.window_left,
                          w.window_right, w.torch_dtype, w.name)


def test_workload_varlen_bf16_d64_w1024_full():
    w = inputs.WORKLOADS["varlen_bf16_d64_w1024"]
    _announce(w.name)
    q, k, v, cu = inputs.make_workload(w)
    o, lse = gpu_varlen(q, k, v, cu, w.causal, w.window_left, w.window_right)
    _check_finite(o, lse)
    check_all_heads_varlen(q, k, v, cu, o, lse, w.softmax_scale, w.causal, w.window_left,
                           w.window_right, w.torch_dtype, w.name)


# ---------------------------------------------------------------------------------------------
# Properties that hold at any size
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("growth", [3.0, 12.0])
@pytest.mark.parametrize("dtype", list(DTYPES))
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mask", ["none", "causal", "window_50_20"])
def test_scores_growing_along_keys(d, dtype, mask, growth):
    """Scores that rise from key tile to key tile (about `growth` log2 units per 64 keys), so
    that the running reference lags the row max: at 3 the new weights stay below the per-lane
    limit without a move (they reach 2^3 and more), at 12 every tile moves the reference.  Both
    must give the oracle's result."""
    _announce(f"growing scores d={d} {dtype} {mask} growth={growth}")
    m = MASKS[mask]
    n = 700
    gen = torch.Generator("cpu").manual_seed(4242 + d)
    q = 0.25 * torch.randn(1, 2, n, d, generator=gen)
    q[..., 0] = 1.0
    k = 0.25 * torch.randn(1, 2, n, d, generator=gen)
    # S[i, j] = scale * q_i . k_j grows by `growth` log2 units per 64 keys through column 0
    scale = 1 / math.sqrt(d)
    k[..., 0] = torch.arange(n, dtype=torch.float32) * (growth / 64 / scale / math.log2(math.e))
    v = torch.randn(1, 2, n, d, generator=gen)
    q, k, v = (x.to(DTYPES[dtype]) for x in (q, k, v))
    o, lse = gpu_dense(q, k, v, m["causal"], m["wl"], m["wr"])
    o_ref, lse_ref = oracle_dense(q, k, v, scale, m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, DTYPES[dtype],
                 f"growing d={d} {dtype} {mask} growth={growth}")


@pytest.mark.parametrize("mask", ["causal", "causal_w37", "window_50_20"])
def test_zero_q_gives_log_count(mask):
    """Q = 0: every visible score is 0, so LSE_i = log(#visible keys of row i) and O_i is the
    mean of the visible V rows (exact mask geometry at full tile counts)."""
    _announce(f"zero q {mask}")
    m = MASKS[mask]
    n, d = 2048, 128
    _, k, v = inputs.make_dense(1, 2, n, d, "bf16", seed=12)
    q = torch.zeros_like(k)
    o, lse = gpu_dense(q, k, v, m["causal"], m["wl"], m["wr"])
    vis = oracle.visibility(n, n, m["causal"], m["wl"], m["wr"])
    cnt = vis.sum(axis=1)
    assert np.allclose(to64(lse[0, 0]), np.log(cnt), atol=1e-5, rtol=0)
    vm = v[0, 0].double().numpy()
    ref = (vis @ vm) / cnt[:, None]
    assert float(np.max(np.abs(to64(o[0, 0]) - ref))) <= O_TOL[torch.bfloat16]


def test_constant_v_gives_constant_output():
    _announce("constant v")
    q, k, _ = inputs.make_dense(1, 2, 1000, 128, "fp16", seed=13)
    v = torch.full_like(q, 0.375)
    o, _ = gpu_dense(q, k, v, True)
    # P is rounded to fp16 for the PV product while l sums the fp32 weights, so O is 0.375
    # up to that rounding, inside the fp16 parity bar
    assert float((o.cpu().double() - 0.375).abs().max()) <= O_TOL[torch.float16]


def test_causal_row_zero_is_v_row_zero():
    _announce("causal row 0")
    q, k, v = inputs.make_dense(2, 2, 777, 64, "bf16", seed=14)
    o, lse = gpu_dense(q, k, v, True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    s00 = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) * float(np.float32(1 / 8))
    assert np.allclose(to64(lse[:, :, 0]), s00.numpy(), atol=1e-5)


def test_deterministic_and_lse_optional():
    _announce("determinism")
    q, k, v = inputs.make_dense(1, 4, 1500, 128, "bf16", seed=15)
    dev = torch.device("cuda:0")
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = attn_fwd(q, k, v, causal=True)
    o2, l2 = attn_fwd(q, k, v, causal=True)
    o3, l3 = attn_fwd(q, k, v, causal=True, return_lse=False)
    torch.cuda.synchronize()
    assert l3 is None
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)


def test_binding_errors_on_gpu_tensors():
    dev = torch.device("cuda:0")
    x = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device=dev)
    with pytest.raises(AttnError, match="HEAD_DIM"):
        attn_fwd(x, x, x)
    y = torch.zeros(1, 1, 8, 64, dtype=torch.float32, device=dev)
    with pytest.raises(AttnError, match="dtype"):
        attn_fwd(y, y, y)
    z = torch.zeros(2, 8, 64, dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 8], dtype=torch.int32, device=dev)
    with pytest.raises(AttnError, match="INVALID_ARG"):
        attn_fwd_varlen(z, z, z, cu, max_seqlen=9)


# Masked dense grids whose (batch, head) pairs split into work-order groups of G > 1 pairs
# with a smaller last group (G = min(ceil(pairs / 8), ceil(32 / q-tiles per head))):
#   B1 H13 N300 d64: 13 pairs, 3 tiles of 128 rows -> G = 2, groups 2,2,2,2,2,2,1
#   B3 H3 N1000 d128 (generic kernel, 36 big tiles): 9 pairs, 8 tiles -> G = 2, last group 1
@pytest.mark.parametrize("shape", [(1, 13, 300, 64), (3, 3, 1000, 128)])
@pytest.mark.parametrize("mask", ["causal", "causal_w37"])
def test_dense_masked_grid_with_partial_last_group(shape, mask):
    b, h, n, d = shape
    _announce(f"dense grouped order {shape} {mask}")
    m = MASKS[mask]
    q, k, v = inputs.make_dense(b, h, n, d, "bf16", seed=300 + h + d)
    o, lse = gpu_dense(q, k, v, m["causal"], m["wl"], m["wr"])
    o_ref, lse_ref = oracle_dense(q, k, v, 1 / math.sqrt(d), m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"{shape} {mask}")


def test_pingpong_masked_grid_with_partial_last_group():
    """B1 H50 N2048 d128 causal: 400 big tiles (ping-pong kernel), 8 tiles per head -> groups of
    G = 4 pairs with a last group of 2.  Heads from the first, a middle and the last group are
    compared with the oracle."""
    _announce("ping-pong grouped order B1 H50 N2048 causal")
    q, k, v = inputs.make_dense(1, 50, 2048, 128, "bf16", seed=350)
    o, lse = gpu_dense(q, k, v, True)
    for hd in (0, 3, 25, 47, 48, 49):
        sl = slice(hd, hd + 1)
        o_ref, lse_ref = oracle_dense(q[:, sl], k[:, sl], v[:, sl], 1 / math.sqrt(128), True,
                                      -1, -1)
        assert_close(to64(o[:, sl]), to64(lse[:, sl]), o_ref, lse_ref, torch.bfloat16,
                     f"head {hd}")


def test_pingpong_causal_odd_tile_count():
    """B1 H256 N2304 d128 causal: 9 q-tiles of 256 rows per head (2304 slots, 9 per workgroup
    of the persistent grid, whose rounds alternate direction so that heavy and light tiles
    pair up).  Work-order groups of 7 heads end in a group of 4.  Heads from the first, a
    middle and the last group are compared with the oracle in full."""
    _announce("ping-pong causal B1 H256 N2304")
    q, k, v = inputs.make_dense(1, 256, 2304, 128, "bf16", seed=360)
    o, lse = gpu_dense(q, k, v, True)
    for hd in (0, 6, 7, 130, 251, 252, 255):
        sl = slice(hd, hd + 1)
        o_ref, lse_ref = oracle_dense(q[:, sl], k[:, sl], v[:, sl], 1 / math.sqrt(128), True,
                                      -1, -1)
        assert_close(to64(o[:, sl]), to64(lse[:, sl]), o_ref, lse_ref, torch.bfloat16,
                     f"head {hd}")
