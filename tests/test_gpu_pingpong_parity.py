"""GPU parity of the d = 128 ping-pong kernel in the configurations the other tests reach
only with bf16 or one-sided masks: fp16 I/O (unmasked, causal, causal with a
left window) and two-sided windows with causal = 0 (both dtypes).  Every grid here is large
enough for the library to pick the ping-pong kernel (256 unmasked / 384 masked 256-row tiles;
the host mirror of that choice in bench.py is asserted first), and every row of every head is
compared with the fp64 oracle.

The two-sided window follows the local branch of `mma` on page
"mainloop_bwd_sm90_tma_gmma_ws.hpp": key j is visible to query i iff
i - window_left <= j <= i + window_right."""

import math

import pytest
import torch

import bench
from exact_attention_49_amd import inputs
from tests.gpu_helpers import check_all_heads_dense, gpu_dense

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}

# name: (batch, heads, seqlen, dtype, causal, window_left, window_right, value_scale)
CASES = {
    # 256 unmasked tiles
    "fp16_none_b1h32n2048": (1, 32, 2048, "fp16", False, -1, -1, 1.0),
    # 1024 causal tiles, four per workgroup of the persistent grid
    "fp16_causal_b2h32n4096": (2, 32, 4096, "fp16", True, -1, -1, 0.5),
    # 384 tiles under a causal mask with a left window (window mask mode)
    "fp16_causal_w300_b1h48n2048": (1, 48, 2048, "fp16", True, 300, -1, 1.0),
    # two-sided windows without causal, 384 and 512 tiles
    "bf16_window_30_70_b1h48n2048": (1, 48, 2048, "bf16", False, 30, 70, 1.0),
    "fp16_window_30_70_b1h48n2048": (1, 48, 2048, "fp16", False, 30, 70, 1.0),
    "bf16_window_500_200_b2h16n4096": (2, 16, 4096, "bf16", False, 500, 200, 1.0),
    "fp16_window_50_20_b1h32n4097": (1, 32, 4097, "fp16", False, 50, 20, 1.0),
}


def _workload(name, b, h, n, dt, causal, wl, wr, vs):
    return inputs.Workload(name=name, batch=b, heads=h, seqlen=n, head_dim=128, dtype=dt,
                           causal=causal, seed=0, window_left=wl, window_right=wr,
                           value_scale=vs)


def test_cases_reach_the_pingpong_kernel():
    for name, c in CASES.items():
        assert bench.kernel_name(_workload(name, *c)) == "attn_fwd_pp_kernel", name


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_pingpong_parity(name):
    b, h, n, dt, causal, wl, wr, vs = CASES[name]
    print(f"[case] ping-pong {name}", flush=True)
    q, k, v = inputs.make_dense(b, h, n, 128, dt, seed=7000 + h + n, value_scale=vs)
    o, lse = gpu_dense(q, k, v, causal, wl, wr)
    check_all_heads_dense(q, k, v, o, lse, 1 / math.sqrt(128), causal, wl, wr, DTYPES[dt], name)
