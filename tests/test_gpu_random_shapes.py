"""GPU parity of seeded random configurations against the fp64 oracle.

Each case draws, from a fixed seed, a head dim (64, 128, 256 or 512), an I/O dtype, query and
K/V head counts (grouped-query groups of 1, 2 or 4), a layout (dense batches with any
sequence length, or packed batches of ragged, possibly empty sequences), a mask mode (none,
causal, causal with a left window, or a two-sided window without causal) and an entry point
(the plain forward, or split-KV with an automatic or explicit split count).  Every row of
every head is compared with the oracle at the forward's bars (O element-wise per dtype, LSE to
1e-3 * max(1, |LSE|)).  The sizes keep each case to a few seconds of oracle time; the draws
cover combinations that the hand-picked cases do not list."""

import math

import numpy as np
import pytest
import torch

from exact_attention_49_amd import (attn_fwd_gqa, attn_fwd_splitkv, attn_fwd_varlen_gqa,
                                    attn_fwd_varlen_splitkv, inputs)
from tests.gpu_helpers import check_all_heads_dense, check_all_heads_varlen

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
N_CASES = 64


def _draw(i):
    rng = np.random.default_rng(20260 + i)
    d = int(rng.choice([64, 128, 256, 512]))
    dt = str(rng.choice(["bf16", "fp16"]))
    hkv = int(rng.integers(1, 4))
    hq = hkv * int(rng.choice([1, 2, 4]))
    mode = int(rng.integers(0, 4))
    causal, wl, wr = [(False, -1, -1), (True, -1, -1),
                      (True, int(rng.integers(0, 400)), -1),
                      (False, int(rng.integers(0, 300)), int(rng.integers(0, 300)))][mode]
    split = int(rng.choice([-1, -1, 0, 2, 5]))  # -1: plain forward, 0: automatic split count
    if bool(rng.integers(0, 2)):
        lens = rng.integers(0, 700, size=int(rng.integers(1, 5))).tolist()
        return dict(d=d, dt=dt, hq=hq, hkv=hkv, causal=causal, wl=wl, wr=wr, split=split,
                    lens=[int(x) for x in lens])
    return dict(d=d, dt=dt, hq=hq, hkv=hkv, causal=causal, wl=wl, wr=wr, split=split,
                batch=int(rng.integers(1, 3)), n=int(rng.integers(1, 900)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    c = _draw(i)
    print(f"[case] random {i}: {c}", flush=True)
    scale = 1 / math.sqrt(c["d"])
    m = dict(causal=c["causal"], window_left=c["wl"], window_right=c["wr"])
    if "lens" in c:
        lens = c["lens"]
        q, k, v, cu = inputs.make_varlen(len(lens), 0, 0, c["hq"], c["d"], c["dt"], seed=9100 + i,
                                         lengths=lens, heads_kv=c["hkv"])
        if int(cu[-1]) == 0:
            pytest.skip("every drawn sequence is empty")
        args = (q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(max(lens), 1))
        if c["split"] >= 0:
            o, lse = attn_fwd_varlen_splitkv(*args, num_splits=c["split"], **m)
        else:
            o, lse = attn_fwd_varlen_gqa(*args, **m)
        torch.cuda.synchronize()
        check_all_heads_varlen(q, k, v, cu, o, lse, scale, c["causal"], c["wl"], c["wr"],
                               DTYPES[c["dt"]], f"random {i}")
    else:
        q, k, v = inputs.make_dense(c["batch"], c["hq"], c["n"], c["d"], c["dt"], seed=9100 + i,
                                    heads_kv=c["hkv"])
        args = (q.to(DEV), k.to(DEV), v.to(DEV))
        if c["split"] >= 0:
            o, lse = attn_fwd_splitkv(*args, num_splits=c["split"], **m)
        else:
            o, lse = attn_fwd_gqa(*args, **m)
        torch.cuda.synchronize()
        check_all_heads_dense(q, k, v, o, lse, scale, c["causal"], c["wl"], c["wr"],
                              DTYPES[c["dt"]], f"random {i}")
