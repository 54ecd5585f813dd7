"""GPU parity of the split-KV entry points (through the C ABI) against the fp64 CPU oracle.

Split-KV computes the same function as the plain path, so the oracle is the same; the cases
cover every head dim, the mask modes, explicit split counts (including more splits than key
tiles, so that some splits are empty), both orders of a causal grid's items over the XCDs,
packed batches, the automatic count, and the low-occupancy workload at full size."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_49_amd import (attn_fwd_splitkv, attn_fwd_varlen_splitkv, inputs,
                                    splitkv_num_splits, splitkv_workspace_size)
from tests.gpu_helpers import (assert_close, check_all_heads_dense, gpu_dense, oracle_dense,
                                to64)

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
MASKS = {
    "none": dict(causal=False, wl=-1, wr=-1),
    "causal": dict(causal=True, wl=-1, wr=-1),
    "window_50_20": dict(causal=False, wl=50, wr=20),
}
DEV = torch.device("cuda:0")


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _split_dense(q, k, v, causal, wl, wr, num_splits, workspace=None):
    o, lse = attn_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_left=wl,
                              window_right=wr, num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("dtype", list(DTYPES))
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_dense_split_all_modes(d, dtype, mask, splits):
    _announce(f"split dense d={d} {dtype} {mask} s={splits}")
    m = MASKS[mask]
    q, k, v = inputs.make_dense(1, 2, 300, d, dtype, seed=500 + d)
    o, lse = _split_dense(q, k, v, m["causal"], m["wl"], m["wr"], splits)
    o_ref, lse_ref = oracle_dense(q, k, v, 1 / math.sqrt(d), m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, DTYPES[dtype],
                 f"split d={d} {dtype} {mask} s={splits}")


@pytest.mark.parametrize("n", [1, 33, 64, 65, 257])
def test_more_splits_than_key_tiles(n):
    # most splits see no key tile at all: they must contribute nothing to the merge
    _announce(f"split n={n} s=16")
    q, k, v = inputs.make_dense(1, 3, n, 128, "bf16", seed=600 + n)
    o, lse = _split_dense(q, k, v, True, -1, -1, 16)
    o_ref, lse_ref = oracle_dense(q, k, v, 1 / math.sqrt(128), True, -1, -1)
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"n={n}")


@pytest.mark.parametrize("b,h", [(1, 1), (1, 3), (2, 2), (4, 3)])
def test_causal_split_work_orders(b, h):
    # causal grids of at most 3 (batch, head) pairs deal their items out to the XCDs one by
    # one, larger ones run contiguous ranges per XCD: both cover every (q-tile, split) once
    _announce(f"causal split order B{b} H{h}")
    q, k, v = inputs.make_dense(b, h, 1100, 128, "bf16", seed=650 + 10 * b + h)
    o, lse = _split_dense(q, k, v, True, -1, -1, 4)
    o_ref, lse_ref = oracle_dense(q, k, v, 1 / math.sqrt(128), True, -1, -1)
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"B{b} H{h}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_empty_splits_ignore_workspace_garbage(d):
    # splits that see no key write LSE = -inf and no partial O: the merge must not read the O
    # left in the workspace (here NaN), which would poison the row through 0 * NaN
    _announce(f"empty splits over a NaN workspace d={d}")
    q, k, v = inputs.make_dense(1, 2, 200, d, "bf16", seed=660 + d)
    nbytes = splitkv_workspace_size(1, 2, 200, d, 12)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    o, lse = _split_dense(q, k, v, True, -1, -1, 12, workspace=ws)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    o_ref, lse_ref = oracle_dense(q, k, v, 1 / math.sqrt(d), True, -1, -1)
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"d={d}")


@pytest.mark.parametrize("d", [64, 128, 512])
def test_split_matches_plain_path(d):
    _announce(f"split vs plain d={d}")
    q, k, v = inputs.make_dense(1, 2, 1000, d, "fp16", seed=700 + d)
    o1, l1 = gpu_dense(q, k, v, True, 300, -1)
    o2, l2 = _split_dense(q, k, v, True, 300, -1, 5)
    assert float((o1.float() - o2.float()).abs().max()) <= 5e-3
    assert float((l1 - l2).abs().max()) <= 1e-4


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mask", ["causal", "window_50_20"])
def test_varlen_split(d, mask):
    _announce(f"split varlen d={d} {mask}")
    m = MASKS[mask]
    lens = [1, 0, 64, 300, 1000, 257, 3]
    q, k, v, cu = inputs.make_varlen(len(lens), 0, 0, 2, d, "bf16", seed=800 + d, lengths=lens)
    o, lse = attn_fwd_varlen_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lens),
                                     causal=m["causal"], window_left=m["wl"],
                                     window_right=m["wr"], num_splits=4)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen(q.float().numpy(), k.float().numpy(),
                                             v.float().numpy(), cu.numpy(), 1 / math.sqrt(d),
                                             m["causal"], m["wl"], m["wr"])
    assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"varlen d={d} {mask}")


def test_workspace_reuse_and_given_buffer():
    # two calls in a row share one caller-owned workspace; the second, smaller one must not
    # see the first one's partial results
    _announce("workspace reuse")
    nbytes = splitkv_workspace_size(1, 2, 2000, 128, 6)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for n in (2000, 700):
        q, k, v = inputs.make_dense(1, 2, n, 128, "bf16", seed=900 + n)
        o, lse = _split_dense(q, k, v, True, -1, -1, 6, workspace=ws)
        o_ref, lse_ref = oracle_dense(q, k, v, 1 / math.sqrt(128), True, -1, -1)
        assert_close(to64(o), to64(lse), o_ref, lse_ref, torch.bfloat16, f"n={n}")


def test_workload_splitkv_bf16_d128_h2_n16384_full():
    """The low-occupancy workload through split-KV with the library's split count: every row
    of both heads against the oracle."""
    w = inputs.WORKLOADS["splitkv_bf16_d128_h2_n16384"]
    _announce(w.name)
    assert splitkv_num_splits(w.batch, w.heads, w.seqlen, w.head_dim, w.causal,
                              w.window_left) > 1
    q, k, v = inputs.make_workload(w)
    o, lse = _split_dense(q, k, v, w.causal, w.window_left, w.window_right, 0)
    check_all_heads_dense(q, k, v, o, lse, w.softmax_scale, w.causal, w.window_left,
                          w.window_right, torch.bfloat16, w.name)
