"""A packed sequence longer than the caller's max_seqlen (a contract violation the host cannot
see, since the lengths live on the device).  The library must neither compute it nor read
past max_seqlen rows of it: every output row of that sequence, in every head, is NaN, and the
other sequences still match the fp64 oracle.  Each entry point that takes max_seqlen is run:
the forward kernels (generic at d = 64/128, ping-pong at d = 128 on a big grid, wide at
d = 512), split-KV with its merge, FP8, and the backward's dQ and dK/dV kernels."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_49_amd import (attn_bwd_varlen, attn_fwd_varlen, attn_fwd_varlen_fp8,
                                    attn_fwd_varlen_splitkv, inputs)
from tests.gpu_helpers import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

LENS = [100, 700, 50, 300]   # the second sequence is longer than the bound below
BOUND = 300
BAD = 1


def _split(cu):
    c = cu.tolist()
    return [(c[s], c[s + 1]) for s in range(len(c) - 1)]


def _check(o, lse, q, k, v, cu, dtype, causal, what):
    o, lse = o.cpu(), (lse.cpu() if lse is not None else None)
    for s, (a, b) in enumerate(_split(cu)):
        if s == BAD:
            assert bool(torch.isnan(o[:, a:b].float()).all()), f"{what}: O of the long sequence"
            if lse is not None:
                assert bool(torch.isnan(lse[:, a:b]).all()), f"{what}: LSE of the long sequence"
            continue
        for h in range(q.shape[0]):
            g = q.shape[0] // k.shape[0]
            o_ref, lse_ref = oracle.attention_head(q[h, a:b].float().numpy(),
                                                   k[h // g, a:b].float().numpy(),
                                                   v[h // g, a:b].float().numpy(),
                                                   1 / math.sqrt(q.shape[-1]), causal)
            assert_close(to64(o[h, a:b]), None if lse is None else to64(lse[h, a:b]), o_ref,
                         lse_ref, dtype, f"{what} seq {s} head {h}")


@pytest.mark.parametrize("d,heads", [(64, 3), (128, 3), (128, 400), (512, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_long_sequence_gives_nan_rows(d, heads, causal):
    print(f"[case] varlen bound d={d} heads={heads} causal={causal}", flush=True)
    q, k, v, cu = inputs.make_varlen(len(LENS), 0, 0, heads, d, "bf16", seed=810 + d,
                                     lengths=LENS)
    o, lse = attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), BOUND, causal=causal)
    torch.cuda.synchronize()
    hs = slice(0, 3)  # the oracle check covers the first heads; NaN rows are checked in all
    assert bool(torch.isnan(o[:, cu[BAD]:cu[BAD + 1]].float()).all())
    _check(o[hs], lse[hs], q[hs], k[hs], v[hs], cu, torch.bfloat16, causal, f"d={d}")


@pytest.mark.parametrize("d", [64, 128, 512])
def test_splitkv_long_sequence_gives_nan_rows(d):
    print(f"[case] varlen bound split-KV d={d}", flush=True)
    q, k, v, cu = inputs.make_varlen(len(LENS), 0, 0, 2, d, "fp16", seed=820 + d,
                                     lengths=LENS)
    o, lse = attn_fwd_varlen_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), BOUND,
                                     causal=True, num_splits=3)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, cu, torch.float16, True, f"split d={d}")


def test_fp8_long_sequence_gives_nan_rows():
    print("[case] varlen bound fp8", flush=True)
    q, k, v, cu = inputs.make_varlen(len(LENS), 0, 0, 2, 128, "bf16", seed=830, lengths=LENS)
    (q8, dq), (k8, dk), (v8, dv) = (inputs.quantize_fp8(x) for x in (q, k, v))
    ds = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in (dq, dk, dv)]
    o, lse = attn_fwd_varlen_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), cu.to(DEV), BOUND,
                                 causal=True, descale_q=ds[0], descale_k=ds[1],
                                 descale_v=ds[2])
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    a, b = _split(cu)[BAD]
    assert bool(torch.isnan(o[:, a:b].float()).all()) and bool(torch.isnan(lse[:, a:b]).all())
    # the other sequences: finite, and the LSE of a sequence's first row is its score with
    # itself (causal), a value the oracle gives exactly
    for s, (a, b) in enumerate(_split(cu)):
        if s != BAD:
            assert bool(torch.isfinite(o[:, a:b].float()).all())
            assert bool(torch.isfinite(lse[:, a:b]).all())


@pytest.mark.parametrize("d", [64, 128])
def test_backward_long_sequence_gives_nan_rows(d):
    print(f"[case] varlen bound backward d={d}", flush=True)
    q, k, v, cu = inputs.make_varlen(len(LENS), 0, 0, 2, d, "bf16", seed=840 + d,
                                     lengths=LENS)
    do = inputs.make_upstream(q.shape, "bf16", seed=841 + d)
    qd, kd, vd, dod, cud = (x.to(DEV) for x in (q, k, v, do, cu))
    # the forward with the true bound, then the backward with the understated one
    o, lse = attn_fwd_varlen(qd, kd, vd, cud, max(LENS), causal=True)
    dq, dk, dv = attn_bwd_varlen(qd, kd, vd, o, lse, dod, cud, BOUND, causal=True)
    torch.cuda.synchronize()
    for s, (a, b) in enumerate(_split(cu)):
        refs = None
        if s != BAD:
            refs = oracle.attention_backward_dense(
                q[None, :, a:b].double().numpy(), k[None, :, a:b].double().numpy(),
                v[None, :, a:b].double().numpy(), do[None, :, a:b].double().numpy(),
                1 / math.sqrt(d), True)
        for gname, g, i in (("dq", dq, 0), ("dk", dk, 1), ("dv", dv, 2)):
            part = g[:, a:b].cpu().double()
            if s == BAD:
                assert bool(torch.isnan(part).all()), gname
            else:
                ref = refs[i][0]
                err = float(np.max(np.abs(part.numpy() - ref)))
                assert err <= 2e-2 * float(np.max(np.abs(ref))), (gname, s, err)
