"""Plain, slow, obviously correct CPU oracle for exact attention forward (fp64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run this
module; it is for the tests, the smoke check and the CPU-baseline leg of the benchmark.
It shares no code with the HIP kernels or their host library.

What it computes.  The pages implement the FlashAttention-2 forward pass (page
"flash_attn_mma_tiling_qk.cu", header comment: Q, K, V, O are [B, H, N, d]; each block takes a
Q tile and streams all of K and V).  Online softmax with rescaling (same page, the "Rescale O"
block: m = max(m_old, m_new), l = exp(m_old - m) * l_old + l_new, O_new = exp(m_old - m_new) *
O_old + P@V, and the final O = O / l) is an exact reorganisation of the plain definition

    S = scale * Q K^T,  S[i, j] = -inf where key j is not visible to query i,
    LSE_i = log sum_j exp(S[i, j])          (natural log)
    O_i = sum_j exp(S[i, j] - LSE_i) V_j

so the oracle is that definition, materialised in float64, one (batch, head) or one
(sequence, head) at a time.  Every function below names the passage it follows.

Visibility (page "mainloop_bwd_sm90_tma_gmma_ws.hpp", the causal masking loop and the local
(sliding-window) branch inside `mma`): with delta = seqlen_k - seqlen_q (bottom-right
alignment), key j is visible to query i iff
    0 <= j < seqlen_k
    and (not causal or j <= i + delta)
    and (window_left  < 0 or j >= i + delta - window_left)
    and (window_right < 0 or j <= i + delta + window_right).
A window bound of -1 means unbounded.  `causal` is the local mask with window_right = 0.

Grouped-query attention: K and V may have fewer heads than Q (a divisor of its head count);
query head h then uses key/value head h // (heads_q // heads_kv) (page
"mainloop_bwd_sm90_tma_gmma_ws.hpp", the qhead_per_khead division).

Empty rows (no visible key): O_i = 0 and LSE_i = -inf (page "flash_fwd_kernel.h" @26a6e0a,
consumer loop: a tile with no key block to visit stores zeros through `store_zero`).

Scale.  The softmax scale is an fp32 argument of the library, so the oracle rounds the given
scale to fp32 first and then works in float64.

All parity functions here are pinned by tests under tests/ (brute force on tiny shapes,
closed forms, invariants and a library routine).  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "visibility",
    "attention_head",
    "attention_dense",
    "attention_varlen",
    "attention_rows_dense",
    "attention_rows_varlen",
    "flops_dense",
    "visible_pairs",
]


def _fp32_scale(scale: float) -> float:
    """The library takes the scale as fp32; the oracle uses that exact value in float64."""
    return float(np.float64(np.float32(scale)))


def _visibility_rows(rows, seqlen_q: int, seqlen_k: int, causal: bool, window_left: int,
                     window_right: int) -> np.ndarray:
    """Visibility of every key to the given query rows (global indices, delta = Nk - Nq)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(seqlen_k, dtype=np.int64)[None, :]
    delta = seqlen_k - seqlen_q
    vis = np.ones((i.shape[0], seqlen_k), dtype=bool)
    if causal:
        vis &= j <= i + delta
    if window_left >= 0:
        vis &= j >= i + delta - window_left
    if window_right >= 0:
        vis &= j <= i + delta + window_right
    return vis


def visibility(seqlen_q: int, seqlen_k: int, causal: bool, window_left: int = -1,
               window_right: int = -1) -> np.ndarray:
    """Boolean [seqlen_q, seqlen_k] matrix: True where key j is visible to query i.

    Follows the causal and local masking predicates of page "mainloop_bwd_sm90_tma_gmma_ws.hpp"
    (`mma`: the separate causal-masking iterations and the Is_local branch), rewritten in
    global indices with delta = seqlen_k - seqlen_q.
    """
    return _visibility_rows(np.arange(seqlen_q), seqlen_q, seqlen_k, causal, window_left,
                            window_right)


def _masked_softmax_times_v(s: np.ndarray, vis: np.ndarray, v: np.ndarray):
    """Rows of scaled scores s with visibility vis -> (O, LSE) by the plain definition.

    LSE_i = m_i + log sum_j exp(s_ij - m_i) over visible j (m_i the row max, which only keeps
    exp in range); P_ij = exp(s_ij - LSE_i) on visible cells, 0 elsewhere; O = P V.
    A row with no visible key gets O = 0 and LSE = -inf.
    """
    s = np.where(vis, s, -np.inf)
    has_any = vis.any(axis=1)
    m = np.where(has_any, np.max(s, axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])                      # exp(-inf) = 0 on masked cells
    denom = np.where(has_any, e.sum(axis=1), 1.0)
    lse = np.where(has_any, m + np.log(denom), -np.inf)
    p = np.where(has_any[:, None], e / denom[:, None], 0.0)
    return p @ v, lse


def attention_head(q, k, v, scale: float, causal: bool = False, window_left: int = -1,
                   window_right: int = -1):
    """One head: q [Nq, d], k [Nk, d], v [Nk, dv] -> (o [Nq, dv] float64, lse [Nq] float64).

    The plain definition of softmax(scale * Q K^T + mask) V with the natural-log LSE of the
    scaled, masked scores; empty rows give O = 0, LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = _fp32_scale(scale) * (q @ k.T)
    vis = visibility(q.shape[0], k.shape[0], causal, window_left, window_right)
    return _masked_softmax_times_v(s, vis, v)


def _kv_group(heads_q: int, heads_kv: int) -> int:
    """Query heads per key/value head.  Grouped-query attention (page
    "mainloop_bwd_sm90_tma_gmma_ws.hpp", the qhead_per_khead division): query head h uses
    key/value head h // group; group 1 is plain multi-head attention."""
    if heads_kv < 1 or heads_q % heads_kv != 0:
        raise ValueError("the key/value head count must divide the query head count")
    return heads_q // heads_kv


def attention_dense(q, k, v, scale: float, causal: bool = False, window_left: int = -1,
                    window_right: int = -1):
    """Dense batch: Q [B, H, N, d], K and V [B, Hkv, N, d] with Hkv dividing H (Hkv = H in
    the plain case; page "flash_attn_mma_tiling_qk.cu", header comment) -> O [B, H, N, d] and
    LSE [B, H, N], both float64."""
    q = np.asarray(q)
    bsz, nh, n, _ = q.shape
    g = _kv_group(nh, np.asarray(k).shape[1])
    dv = np.asarray(v).shape[-1]
    o = np.empty((bsz, nh, n, dv), dtype=np.float64)
    lse = np.empty((bsz, nh, n), dtype=np.float64)
    for b in range(bsz):
        for h in range(nh):
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h // g], v[b, h // g], scale,
                                                causal, window_left, window_right)
    return o, lse


def _check_cu_seqlens(cu_seqlens, total: int) -> np.ndarray:
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != total:
        raise ValueError("cu_seqlens must start at 0, be nondecreasing and end at total_tokens")
    return cu


def attention_varlen(q, k, v, cu_seqlens, scale: float, causal: bool = False,
                     window_left: int = -1, window_right: int = -1):
    """Packed variable-length batch: Q [H, total_tokens, d], K and V [Hkv, total_tokens, d]
    (Hkv dividing H, as in `attention_dense`); sequence s owns tokens
    [cu_seqlens[s], cu_seqlens[s+1]) (page "mainloop_bwd_sm90_tma_gmma_ws.hpp", get_seqlen_q/k:
    the length is the difference of consecutive cu_seqlens entries).  Each sequence attends
    only within itself.  Returns O [H, total, d] and LSE [H, total], float64."""
    q = np.asarray(q)
    nh, total, _ = q.shape
    g = _kv_group(nh, np.asarray(k).shape[0])
    dv = np.asarray(v).shape[-1]
    cu = _check_cu_seqlens(cu_seqlens, total)
    o = np.zeros((nh, total, dv), dtype=np.float64)
    lse = np.zeros((nh, total), dtype=np.float64)
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(nh):
            o[h, a:b], lse[h, a:b] = attention_head(q[h, a:b], k[h // g, a:b], v[h // g, a:b],
                                                    scale, causal, window_left, window_right)
    return o, lse


def _rows_one_head(q, k, v, rows, scale, causal, wl, wr):
    """O and LSE of selected query rows of one head: the same definition restricted to those
    rows (the visibility of row i depends only on i, Nq and Nk)."""
    q = np.asarray(q)
    s = _fp32_scale(scale) * (np.asarray(q[rows], dtype=np.float64)
                              @ np.asarray(k, dtype=np.float64).T)
    vis = _visibility_rows(rows, q.shape[0], k.shape[0], causal, wl, wr)
    return _masked_softmax_times_v(s, vis, np.asarray(v, dtype=np.float64))


def attention_rows_dense(q, k, v, index, scale: float, causal: bool = False,
                         window_left: int = -1, window_right: int = -1):
    """O and LSE for sampled rows of a dense batch, for shapes too large to materialise whole.

    `index` is an int array [R, 3] of (b, h, i).  Same definition as `attention_dense`,
    evaluated only at the requested rows.  Returns (o [R, d], lse [R]) float64."""
    idx = np.asarray(index, dtype=np.int64).reshape(-1, 3)
    q = np.asarray(q)
    g = _kv_group(q.shape[1], np.asarray(k).shape[1])
    o = np.empty((idx.shape[0], np.asarray(v).shape[-1]), dtype=np.float64)
    lse = np.empty(idx.shape[0], dtype=np.float64)
    for (b, h) in sorted({(int(b), int(h)) for b, h, _ in idx}):
        sel = np.nonzero((idx[:, 0] == b) & (idx[:, 1] == h))[0]
        o[sel], lse[sel] = _rows_one_head(q[b, h], k[b, h // g], v[b, h // g], idx[sel, 2],
                                          scale, causal, window_left, window_right)
    return o, lse


def attention_rows_varlen(q, k, v, cu_seqlens, index, scale: float, causal: bool = False,
                          window_left: int = -1, window_right: int = -1):
    """O and LSE for sampled rows of a packed batch.  `index` is [R, 2] of (h, token).
    Same definition as `attention_varlen`, evaluated only at the requested rows."""
    idx = np.asarray(index, dtype=np.int64).reshape(-1, 2)
    q = np.asarray(q)
    g = _kv_group(q.shape[0], np.asarray(k).shape[0])
    cu = _check_cu_seqlens(cu_seqlens, q.shape[1])
    o = np.empty((idx.shape[0], np.asarray(v).shape[-1]), dtype=np.float64)
    lse = np.empty(idx.shape[0], dtype=np.float64)
    seq_of = np.searchsorted(cu, idx[:, 1], side="right") - 1
    for (h, s) in sorted({(int(h), int(s)) for h, s in zip(idx[:, 0], seq_of)}):
        sel = np.nonzero((idx[:, 0] == h) & (seq_of == s))[0]
        a, b = int(cu[s]), int(cu[s + 1])
        o[sel], lse[sel] = _rows_one_head(q[h, a:b], k[h // g, a:b], v[h // g, a:b],
                                          idx[sel, 1] - a, scale, causal, window_left,
                                          window_right)
    return o, lse


def visible_pairs(seqlen: int, causal: bool, window_left: int = -1, window_right: int = -1) -> int:
    """Exact number of visible (query, key) pairs of one head of one sequence (Nq = Nk)."""
    total = 0
    for i in range(seqlen):
        lo = 0
        hi = seqlen - 1
        if causal:
            hi = min(hi, i)
        if window_left >= 0:
            lo = max(lo, i - window_left)
        if window_right >= 0:
            hi = min(hi, i + window_right)
        total += max(0, hi - lo + 1)
    return total


def flops_dense(batch: int, heads: int, seqlen: int, head_dim: int, causal: bool) -> float:
    """The benchmark's FLOP count: 4 * B * H * N^2 * d (two N x N x d products), halved when
    causal."""
    f = 4.0 * batch * heads * seqlen * seqlen * head_dim
    return f / 2 if causal else f
