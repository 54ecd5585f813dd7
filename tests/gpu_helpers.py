"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and compare it
element by element with the fp64 CPU oracle."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from exact_attention_49_amd import attn_fwd, attn_fwd_varlen

# Parity bars: max |O_gpu - O_ref| per I/O dtype; LSE within 1e-3 relative, with a unit floor
# (|d| <= 1e-3 * max(1, |ref|)) since causal row 0 has LSE = s_00, which may be near zero.
O_TOL = {torch.bfloat16: 2e-2, torch.float16: 5e-3}
LSE_REL = 1e-3


def gpu_dense(q, k, v, causal=False, wl=-1, wr=-1, scale=None):
    dev = torch.device("cuda:0")
    o, lse = attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, window_left=wl,
                      window_right=wr, softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


def gpu_varlen(q, k, v, cu, causal=False, wl=-1, wr=-1, scale=None):
    dev = torch.device("cuda:0")
    lens = (cu[1:] - cu[:-1]).tolist()
    o, lse = attn_fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev),
                             max(max(lens), 1), causal=causal, window_left=wl, window_right=wr,
                             softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


def to64(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float64).numpy()


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Element-wise parity of O and LSE (numpy float64 arrays of equal shape)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    err = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    assert err <= O_TOL[dtype], f"{what}: max|dO| = {err:.3e} > {O_TOL[dtype]}"
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        fin = np.isfinite(lse_ref)
        assert np.all(lse_gpu[~fin] == -np.inf), f"{what}: empty rows must give -inf"
        d = np.abs(lse_gpu[fin] - lse_ref[fin])
        bound = LSE_REL * np.maximum(1.0, np.abs(lse_ref[fin]))
        assert np.all(d <= bound), f"{what}: LSE err {float(np.max(d / bound)):.3f} x bound"
    return err


def sample_rows(n: int, rng: np.random.Generator, extra: int = 8):
    """Rows at tile boundaries, both ends and a few random ones."""
    rows = {0, 1, n - 1, n - 2}
    for t in (31, 32, 63, 64, 127, 128, 255, 256, 511, 512, 1023, 1024, 1025):
        if t < n:
            rows.add(t)
    rows.update(int(x) for x in rng.integers(0, n, extra))
    return sorted(r for r in rows if 0 <= r < n)


def softmax_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def oracle_dense(q, k, v, scale, causal, wl, wr):
    return oracle.attention_dense(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                  scale, causal, wl, wr)


def _oracle_workers() -> int:
    # the oracle's elementwise passes run on one core; BLAS threads share the rest
    import os
    return max(1, min(8, (os.cpu_count() or 2) // 2))


def check_all_heads_dense(q, k, v, o, lse, scale, causal, wl, wr, dtype, what=""):
    """Every row of every (batch, head) of a dense result against the oracle, one head per
    oracle call (query head h reads K/V head h // (H / Hkv)); heads run in a thread pool.
    q, k, v are the CPU inputs, o and lse the GPU outputs (any device).  Returns the largest
    O error."""
    from concurrent.futures import ThreadPoolExecutor

    o, lse = o.cpu(), lse.cpu() if lse is not None else None
    bsz, nh = q.shape[0], q.shape[1]
    g = nh // k.shape[1]
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()

    def one(bh):
        b, h = bh
        o_ref, lse_ref = oracle.attention_head(qf[b, h], kf[b, h // g], vf[b, h // g], scale,
                                               causal, wl, wr)
        return assert_close(to64(o[b, h]), None if lse is None else to64(lse[b, h]), o_ref,
                            lse_ref, dtype, f"{what} b={b} h={h}")

    pairs = [(b, h) for b in range(bsz) for h in range(nh)]
    with ThreadPoolExecutor(_oracle_workers()) as ex:
        errs = list(ex.map(one, pairs))
    return max(errs)


def check_all_heads_varlen(q, k, v, cu, o, lse, scale, causal, wl, wr, dtype, what=""):
    """Every row of every (sequence, head) of a packed result against the oracle, one
    (sequence, head) per oracle call, in a thread pool.  Returns the largest O error."""
    from concurrent.futures import ThreadPoolExecutor

    o, lse = o.cpu(), lse.cpu() if lse is not None else None
    nh = q.shape[0]
    g = nh // k.shape[0]
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    cu_l = [int(x) for x in cu.tolist()]

    def one(sh):
        s, h = sh
        a, b = cu_l[s], cu_l[s + 1]
        o_ref, lse_ref = oracle.attention_head(qf[h, a:b], kf[h // g, a:b], vf[h // g, a:b],
                                               scale, causal, wl, wr)
        return assert_close(to64(o[h, a:b]), None if lse is None else to64(lse[h, a:b]), o_ref,
                            lse_ref, dtype, f"{what} seq={s} h={h}")

    jobs = [(s, h) for s in range(len(cu_l) - 1) if cu_l[s + 1] > cu_l[s] for h in range(nh)]
    with ThreadPoolExecutor(_oracle_workers()) as ex:
        errs = list(ex.map(one, jobs))
    return max(errs) if errs else 0.0
