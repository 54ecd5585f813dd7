"""Plain, slow, obviously correct CPU oracle for the exact-attention backward pass (fp64).

TEST INFRASTRUCTURE ONLY, like oracle/attention.py: nothing on the product path may import,
call or run it.  It shares no code with the HIP kernels or their host library.

What it computes.  For the forward O = P V with P = softmax(S) row by row over the visible
keys and S = scale * Q K^T, the gradients of a loss with upstream gradient dO = dL/dO are
(page "mainloop_bwd_sm90_tma_gmma_ws.hpp", the backward `mma`: P is recomputed from S and
the stored LSE; dP = dO V^T; dS = P * (dP - dPsum) elementwise with dPsum one value per query
row; dV accumulates P^T dO, dK accumulates dS^T Q and is multiplied by the softmax scale at
the end; dQ accumulates dS K, to which the scale applies the same way):

    P_ij   = exp(S_ij - LSE_i) on visible cells, 0 elsewhere
    dV     = P^T dO
    dP     = dO V^T
    dPsum_i = sum_j P_ij dP_ij
    dS     = P * (dP - dPsum[:, None])
    dQ     = scale * dS K
    dK     = scale * dS^T Q

The pages take dPsum as an input and do not show how it is formed; the oracle uses its
definition above, the row sum of P * dP (the softmax Jacobian's diagonal correction).  It
equals dO_i . O_i, since O_i = sum_j P_ij V_j; a test checks that identity.

Grouped-query attention: query head h uses key/value head h // (Hq // Hkv), so the dK and dV
of a key/value head are the sums of the contributions of the query heads of its group.
A query row with no visible key has P = 0 and contributes nothing.

Every function here is pinned by tests under tests/ (torch's float64 autograd, central finite
differences of the forward oracle, closed forms and invariants).  None is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

from .attention import _check_cu_seqlens, _fp32_scale, _kv_group, visibility

__all__ = [
    "attention_head_backward",
    "attention_backward_dense",
    "attention_backward_varlen",
    "flops_backward_dense",
]


def attention_head_backward(q, k, v, do, scale: float, causal: bool = False,
                            window_left: int = -1, window_right: int = -1):
    """One head: q, do [Nq, d], k, v [Nk, d] -> (dq, dk, dv) float64, by the definitions in
    the module docstring, with P materialised from the scaled, masked scores."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    sc = _fp32_scale(scale)
    vis = visibility(q.shape[0], k.shape[0], causal, window_left, window_right)
    s = np.where(vis, sc * (q @ k.T), -np.inf)
    has_any = vis.any(axis=1)
    m = np.where(has_any, np.max(s, axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])
    denom = np.where(has_any, e.sum(axis=1), 1.0)
    p = np.where(has_any[:, None], e / denom[:, None], 0.0)
    dv = p.T @ do
    dp = do @ v.T
    dpsum = np.sum(p * dp, axis=1)
    ds = p * (dp - dpsum[:, None])
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


def attention_backward_dense(q, k, v, do, scale: float, causal: bool = False,
                             window_left: int = -1, window_right: int = -1):
    """Dense batch: q, do [B, H, N, d]; k, v [B, Hkv, N, d] with Hkv dividing H.
    Returns dq [B, H, N, d] and dk, dv [B, Hkv, N, d], float64."""
    q, do = np.asarray(q), np.asarray(do)
    k, v = np.asarray(k), np.asarray(v)
    bsz, nh = q.shape[:2]
    g = _kv_group(nh, k.shape[1])
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(bsz):
        for h in range(nh):
            gq, gk, gv = attention_head_backward(q[b, h], k[b, h // g], v[b, h // g], do[b, h],
                                                 scale, causal, window_left, window_right)
            dq[b, h] = gq
            dk[b, h // g] += gk
            dv[b, h // g] += gv
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_seqlens, scale: float, causal: bool = False,
                              window_left: int = -1, window_right: int = -1):
    """Packed batch: q, do [H, total, d]; k, v [Hkv, total, d]; sequence s owns tokens
    [cu[s], cu[s+1]) and attends only within itself.  Returns dq [H, total, d] and dk, dv
    [Hkv, total, d], float64."""
    q, do = np.asarray(q), np.asarray(do)
    k, v = np.asarray(k), np.asarray(v)
    nh, total = q.shape[:2]
    g = _kv_group(nh, k.shape[0])
    cu = _check_cu_seqlens(cu_seqlens, total)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        for h in range(nh):
            gq, gk, gv = attention_head_backward(q[h, a:b], k[h // g, a:b], v[h // g, a:b],
                                                 do[h, a:b], scale, causal, window_left,
                                                 window_right)
            dq[h, a:b] = gq
            dk[h // g, a:b] += gk
            dv[h // g, a:b] += gv
    return dq, dk, dv


def flops_backward_dense(batch: int, heads: int, seqlen: int, head_dim: int,
                         causal: bool) -> float:
    """The usual backward FLOP count: five N x N x d products (S, dP, dV, dK, dQ), i.e. 2.5
    times the forward's 4 * B * H * N^2 * d, halved when causal."""
    f = 10.0 * batch * heads * seqlen ** 2 * head_dim
    return f / 2 if causal else f
