"""Pins for the fp64 CPU oracle: each test checks it against something other than itself.

- a scalar brute force that follows the pages' streaming recurrence one key at a time (page
  "flash_attn_mma_tiling_qk.cu", the online rescale block: m = max(m_old, m_new),
  l = exp(m_old - m) l_old + rowsum(P), O = exp(m_old - m) O_old + P V, O /= l at the end) with
  visibility taken from the tile-local masking predicates of page
  "mainloop_bwd_sm90_tma_gmma_ws.hpp" (`mma`, causal masking iterations and Is_local branch);
- hand-derived values (tests/golden/hand_softmax_cases.json);
- closed forms (Q = 0 gives LSE = log #visible and O = mean of visible V; causal row 0);
- invariants (rows of P sum to one, constant V, permutation equivariance, scale covariance,
  a window wider than N equals plain causal, a packed batch equals its sequences run alone);
- a library routine (torch's float64 CPU scaled_dot_product_attention with a boolean mask).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_49_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_softmax_cases.json")
BIG = 1 << 30


# ---------------------------------------------------------------------------------------------
# Independent formulations used only as pins
# ---------------------------------------------------------------------------------------------

def page_tile_mask(seqlen_q, seqlen_k, causal, wl, wr, block_m, block_n):
    """Visibility from the tile-local predicates on page "mainloop_bwd_sm90_tma_gmma_ws.hpp".

    For tile (m_block, n_block) and in-tile indices (k_local, q_local):
      causal:     masked iff k_local >= min(q_local + 1 + Nk - n*BN - Nq + m*BM, Nk - n*BN)
      local:      masked iff k_local >= min(q_local + 1 + Nk - n*BN - Nq + m*BM + wr, Nk - n*BN)
                          or k_local <  max(q_local + Nk - n*BN - Nq + m*BM - wl, 0)
      otherwise:  masked iff k_local >= Nk - n*BN
    Causal with a left window is the local case with wr = 0; an unbounded side is a huge bound.
    """
    local = wl >= 0 or (wr >= 0 and not causal)
    if local:
        wl_ = wl if wl >= 0 else BIG
        wr_ = 0 if causal else (wr if wr >= 0 else BIG)
    vis = [[False] * seqlen_k for _ in range(seqlen_q)]
    for m in range((seqlen_q + block_m - 1) // block_m):
        for n in range((seqlen_k + block_n - 1) // block_n):
            for ql in range(block_m):
                for kl in range(block_n):
                    qi, kj = m * block_m + ql, n * block_n + kl
                    if qi >= seqlen_q or kj >= seqlen_k:
                        continue
                    lim = seqlen_k - n * block_n
                    if local:
                        right = 1 + seqlen_k - n * block_n - seqlen_q + m * block_m + wr_
                        left = seqlen_k - n * block_n - seqlen_q + m * block_m - wl_
                        masked = kl >= min(ql + right, lim) or kl < max(ql + left, 0)
                    elif causal:
                        off = 1 + seqlen_k - n * block_n - seqlen_q + m * block_m
                        masked = kl >= min(ql + off, lim)
                    else:
                        masked = kl >= lim
                    vis[qi][kj] = not masked
    return vis


def brute_force(q, k, v, scale, vis):
    """Scalar streaming softmax, one key at a time, in Python floats."""
    scale = float(np.float32(scale))
    nq, dv = len(q), len(v[0])
    out, lse = [], []
    for i in range(nq):
        m, l, acc = -math.inf, 0.0, [0.0] * dv
        for j in range(len(k)):
            if not vis[i][j]:
                continue
            s = scale * sum(a * b for a, b in zip(q[i], k[j]))
            m_new = max(m, s)
            alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
            p = math.exp(s - m_new)
            l = alpha * l + p
            acc = [alpha * a + p * x for a, x in zip(acc, v[j])]
            m = m_new
        if l == 0.0:
            out.append([0.0] * dv)
            lse.append(-math.inf)
        else:
            out.append([a / l for a in acc])
            lse.append(m + math.log(l))
    return np.array(out), np.array(lse)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


MASKS = [
    dict(causal=False, wl=-1, wr=-1),
    dict(causal=True, wl=-1, wr=-1),
    dict(causal=True, wl=3, wr=-1),
    dict(causal=False, wl=2, wr=4),
    dict(causal=False, wl=0, wr=0),
    dict(causal=False, wl=-1, wr=1),
    dict(causal=False, wl=5, wr=-1),
]


# ---------------------------------------------------------------------------------------------
# Mask geometry
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("nq,nk", [(13, 13), (7, 11), (11, 7), (16, 16)])
@pytest.mark.parametrize("bm,bn", [(4, 4), (3, 5), (8, 2)])
def test_visibility_matches_page_tile_predicates(mask, nq, nk, bm, bn):
    ref = np.array(page_tile_mask(nq, nk, mask["causal"], mask["wl"], mask["wr"], bm, bn))
    got = oracle.visibility(nq, nk, mask["causal"], mask["wl"], mask["wr"])
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("n", [1, 2, 7, 64, 300])
def test_visible_pairs_counts(n):
    for mask in MASKS:
        vis = oracle.visibility(n, n, mask["causal"], mask["wl"], mask["wr"])
        assert oracle.visible_pairs(n, mask["causal"], mask["wl"], mask["wr"]) == int(vis.sum())
    # closed forms: causal n(n+1)/2; causal window w: sum_i min(i, w) + 1
    assert oracle.visible_pairs(n, True) == n * (n + 1) // 2
    w = 5
    assert oracle.visible_pairs(n, True, w, 0) == sum(min(i, w) + 1 for i in range(n))


# ---------------------------------------------------------------------------------------------
# Whole oracle vs brute force and vs a library routine
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("nq,nk,d,dv", [(9, 9, 4, 4), (16, 16, 8, 3), (5, 12, 3, 6), (12, 5, 2, 2)])
def test_oracle_matches_streaming_brute_force(mask, nq, nk, d, dv):
    q, k, v = rnd((nq, d), 1), rnd((nk, d), 2), rnd((nk, dv), 3)
    scale = 0.7
    vis = page_tile_mask(nq, nk, mask["causal"], mask["wl"], mask["wr"], 4, 4)
    o_ref, lse_ref = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, vis)
    o, lse = oracle.attention_head(q, k, v, scale, mask["causal"], mask["wl"], mask["wr"])
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(lse[~fin] == -np.inf)
    assert np.allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)


def test_varlen_matches_brute_force_three_sequences():
    lens = [5, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    nh, d = 2, 4
    q, k, v = rnd((nh, cu[-1], d), 4), rnd((nh, cu[-1], d), 5), rnd((nh, cu[-1], d), 6)
    for mask in MASKS[:4]:
        o, lse = oracle.attention_varlen(q, k, v, cu, 0.5, mask["causal"], mask["wl"], mask["wr"])
        for s in range(len(lens)):
            a, b = cu[s], cu[s + 1]
            vis = page_tile_mask(b - a, b - a, mask["causal"], mask["wl"], mask["wr"], 2, 3)
            for h in range(nh):
                o_ref, lse_ref = brute_force(q[h, a:b].tolist(), k[h, a:b].tolist(),
                                             v[h, a:b].tolist(), 0.5, vis)
                assert np.allclose(o[h, a:b], o_ref, atol=1e-12, rtol=0)
                assert np.allclose(lse[h, a:b], lse_ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("mask", MASKS)
def test_oracle_matches_torch_sdpa_float64(mask):
    bsz, nh, n, d = 2, 3, 37, 16
    q, k, v = rnd((bsz, nh, n, d), 7), rnd((bsz, nh, n, d), 8), rnd((bsz, nh, n, d), 9)
    scale = float(np.float32(1 / math.sqrt(d)))
    vis = torch.from_numpy(oracle.visibility(n, n, mask["causal"], mask["wl"], mask["wr"]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=vis,
        scale=scale).numpy()
    o, _ = oracle.attention_dense(q, k, v, scale, mask["causal"], mask["wl"], mask["wr"])
    assert np.allclose(o, ref, atol=1e-10, rtol=0)


@pytest.mark.parametrize("mask", MASKS[:4])
@pytest.mark.parametrize("nh,nkv", [(4, 2), (6, 1), (6, 3), (3, 3)])
def test_gqa_matches_torch_sdpa_enable_gqa(mask, nh, nkv):
    """Grouped-query attention against torch's own grouped SDPA (float64, CPU), which gives
    query head h the key/value head h // (H / Hkv), the same grouping as the qhead_per_khead
    division of page "mainloop_bwd_sm90_tma_gmma_ws.hpp"."""
    bsz, n, d = 2, 29, 8
    q, k, v = rnd((bsz, nh, n, d), 11), rnd((bsz, nkv, n, d), 12), rnd((bsz, nkv, n, d), 13)
    scale = 0.3
    vis = torch.from_numpy(oracle.visibility(n, n, mask["causal"], mask["wl"], mask["wr"]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=vis,
        scale=float(np.float32(scale)), enable_gqa=True).numpy()
    o, _ = oracle.attention_dense(q, k, v, scale, mask["causal"], mask["wl"], mask["wr"])
    assert np.allclose(o, ref, atol=1e-10, rtol=0)


def test_gqa_head_mapping_is_grouped_not_strided():
    """With 4 query heads on 2 key/value heads, query heads 0 and 1 share key/value head 0:
    their outputs match the plain attention of that head, and differ from head 1's."""
    q, k, v = rnd((1, 4, 10, 4), 14), rnd((1, 2, 10, 4), 15), rnd((1, 2, 10, 4), 16)
    o, lse = oracle.attention_dense(q, k, v, 0.5, True)
    for h in range(4):
        o_h, lse_h = oracle.attention_head(q[0, h], k[0, h // 2], v[0, h // 2], 0.5, True)
        o_x, _ = oracle.attention_head(q[0, h], k[0, 1 - h // 2], v[0, 1 - h // 2], 0.5, True)
        assert np.array_equal(o[0, h], o_h) and np.array_equal(lse[0, h], lse_h)
        assert not np.allclose(o[0, h], o_x)


def test_gqa_rejects_non_divisor_head_count():
    q, k = rnd((1, 4, 5, 4), 17), rnd((1, 3, 5, 4), 18)
    with pytest.raises(ValueError):
        oracle.attention_dense(q, k, k, 0.5)
    with pytest.raises(ValueError):
        oracle.attention_varlen(q[0], k[0], k[0], np.array([0, 5]), 0.5)


def test_gqa_varlen_and_sampled_rows():
    """Varlen GQA is dense GQA per sequence; sampled rows equal the full result."""
    lens = [9, 0, 14, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qv, kv, vv = rnd((6, cu[-1], 4), 19), rnd((2, cu[-1], 4), 20), rnd((2, cu[-1], 4), 21)
    o, lse = oracle.attention_varlen(qv, kv, vv, cu, 0.6, True, 5, 0)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        od, ld = oracle.attention_dense(qv[None, :, a:b], kv[None, :, a:b], vv[None, :, a:b],
                                        0.6, True, 5, 0)
        assert np.array_equal(o[:, a:b], od[0]) and np.array_equal(lse[:, a:b], ld[0])
    idx = np.array([[0, 0], [5, 8], [2, 9], [3, 22], [4, 26], [1, 13]])
    o_r, lse_r = oracle.attention_rows_varlen(qv, kv, vv, cu, idx, 0.6, True, 5, 0)
    assert np.allclose(o_r, o[idx[:, 0], idx[:, 1]], atol=1e-13)
    assert np.allclose(lse_r, lse[idx[:, 0], idx[:, 1]], atol=1e-13)
    q, k, v = rnd((2, 6, 30, 4), 22), rnd((2, 3, 30, 4), 23), rnd((2, 3, 30, 4), 24)
    o, lse = oracle.attention_dense(q, k, v, 0.6, False, 3, 2)
    idx = np.array([[0, 0, 0], [1, 5, 29], [0, 3, 11], [1, 2, 4]])
    o_r, lse_r = oracle.attention_rows_dense(q, k, v, idx, 0.6, False, 3, 2)
    assert np.allclose(o_r, o[idx[:, 0], idx[:, 1], idx[:, 2]], atol=1e-13)
    assert np.allclose(lse_r, lse[idx[:, 0], idx[:, 1], idx[:, 2]], atol=1e-13)


# ---------------------------------------------------------------------------------------------
# Hand-derived values
# ---------------------------------------------------------------------------------------------

def _lse_value(x):
    if x == "-inf":
        return -math.inf
    assert x.startswith("ln")
    return math.log(float(x[2:]))


def test_golden_hand_derived_cases():
    with open(GOLDEN) as f:
        g = json.load(f)
    inp = g["inputs"]
    q, k, v = (np.array(inp[n]) for n in ("q", "k", "v"))
    for case in g["cases"]:
        o, lse = oracle.attention_head(q, k, v, inp["scale"], case["causal"],
                                       case["window_left"], case["window_right"])
        assert np.allclose(o[:, 0], case["o"], atol=inp["tol"], rtol=0), case["name"]
        assert np.allclose(lse, [_lse_value(x) for x in case["lse"]], atol=inp["tol"], rtol=0)
    e = g["empty_row_case"]
    o, lse = oracle.attention_head(np.array(e["q"]), np.array(e["k"]), np.array(e["v"]), 1.0,
                                   True)
    assert np.allclose(o[:, 0], e["o"], atol=1e-12, rtol=0)
    ref = [_lse_value(x) for x in e["lse"]]
    assert lse[0] == -math.inf and np.allclose(lse[1:], ref[1:], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("mask", MASKS)
def test_softmax_rows_sum_to_one(mask):
    n = 23
    q, k = rnd((n, 8), 10), rnd((n, 8), 11)
    p, _ = oracle.attention_head(q, k, np.eye(n), 0.9, mask["causal"], mask["wl"], mask["wr"])
    vis = oracle.visibility(n, n, mask["causal"], mask["wl"], mask["wr"])
    assert np.all(p >= 0)
    assert np.all(p[~vis] == 0)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12, rtol=0)


@pytest.mark.parametrize("mask", MASKS)
def test_constant_v_gives_constant_output(mask):
    n, d = 31, 8
    q, k = rnd((n, d), 12), rnd((n, d), 13)
    v = np.tile(np.array([1.5, -2.0, 0.25]), (n, 1))
    o, _ = oracle.attention_head(q, k, v, 1.1, mask["causal"], mask["wl"], mask["wr"])
    assert np.allclose(o, v, atol=1e-12, rtol=0)


def _count_closed_form(i, n, causal, wl, wr):
    left = i if wl < 0 else min(i, wl)
    if causal:
        right = 0
    else:
        right = (n - 1 - i) if wr < 0 else min(n - 1 - i, wr)
    return left + right + 1


@pytest.mark.parametrize("mask", MASKS)
def test_zero_q_gives_log_count_and_mean(mask):
    n, d = 40, 4
    q = np.zeros((n, d))
    k, v = rnd((n, d), 14), rnd((n, 5), 15)
    o, lse = oracle.attention_head(q, k, v, 0.3, mask["causal"], mask["wl"], mask["wr"])
    for i in range(n):
        cnt = _count_closed_form(i, n, mask["causal"], mask["wl"], mask["wr"])
        assert abs(lse[i] - math.log(cnt)) < 1e-12
        lo = i - (i if mask["wl"] < 0 else min(i, mask["wl"]))
        assert np.allclose(o[i], v[lo:lo + cnt].mean(axis=0), atol=1e-12, rtol=0)


def test_zero_q_window_1024_reading():
    # the packed workload's window: causal with window_left = 1024 -> 1025 keys per late row
    n = 1500
    q = np.zeros((n, 2))
    k, v = rnd((n, 2), 16), rnd((n, 2), 17)
    _, lse = oracle.attention_head(q, k, v, 1.0, True, 1024, 0)
    assert abs(lse[1024] - math.log(1025)) < 1e-12
    assert abs(lse[1499] - math.log(1025)) < 1e-12
    assert abs(lse[100] - math.log(101)) < 1e-12


def test_permutation_equivariance():
    n, d = 29, 8
    q, k, v = rnd((n, d), 18), rnd((n, d), 19), rnd((n, d), 20)
    o, lse = oracle.attention_head(q, k, v, 0.4)
    perm = np.random.default_rng(21).permutation(n)
    o2, lse2 = oracle.attention_head(q, k[perm], v[perm], 0.4)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
    o3, lse3 = oracle.attention_head(q[perm], k, v, 0.4)
    assert np.allclose(o[perm], o3, atol=1e-12) and np.allclose(lse[perm], lse3, atol=1e-12)


def test_causal_row_zero():
    n, d = 17, 8
    q, k, v = rnd((n, d), 22), rnd((n, d), 23), rnd((n, d), 24)
    scale = 0.125
    o, lse = oracle.attention_head(q, k, v, scale, causal=True)
    assert np.allclose(o[0], v[0], atol=1e-14)
    assert abs(lse[0] - scale * float(q[0] @ k[0])) < 1e-12


def test_scale_covariance():
    n, d = 19, 8
    q, k, v = rnd((n, d), 25), rnd((n, d), 26), rnd((n, d), 27)
    for causal in (False, True):
        o, lse = oracle.attention_head(q, k, v, 0.5, causal)
        o2, lse2 = oracle.attention_head(2.0 * q, k, v, 0.25, causal)
        assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)


def test_scale_is_rounded_to_fp32():
    # the library's scale argument is fp32; 0.1 is not representable, so fp32(0.1) is used
    n, d = 6, 4
    q, k, v = rnd((n, d), 28), rnd((n, d), 29), rnd((n, d), 30)
    o, _ = oracle.attention_head(q, k, v, 0.1)
    o32, _ = oracle.attention_head(q * float(np.float32(0.1)) / 0.5, k, v, 0.5)
    assert np.allclose(o, o32, atol=1e-12)


def test_wide_window_equals_causal():
    n, d = 33, 8
    q, k, v = rnd((n, d), 31), rnd((n, d), 32), rnd((n, d), 33)
    o, lse = oracle.attention_head(q, k, v, 0.3, causal=True)
    o2, lse2 = oracle.attention_head(q, k, v, 0.3, True, n + 5, 0)
    o3, lse3 = oracle.attention_head(q, k, v, 0.3, False, -1, 0)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    assert np.array_equal(o, o3) and np.array_equal(lse, lse3)


def test_varlen_equals_per_sequence_dense():
    q, k, v, cu = inputs.make_varlen(5, 1, 70, 3, 16, "bf16", seed=34)
    qf, kf, vf = (x.float().numpy() for x in (q, k, v))
    cu = cu.numpy()
    o, lse = oracle.attention_varlen(qf, kf, vf, cu, 0.25, True, 9, 0)
    for s in range(5):
        a, b = cu[s], cu[s + 1]
        od, ld = oracle.attention_dense(qf[None, :, a:b], kf[None, :, a:b], vf[None, :, a:b],
                                        0.25, True, 9, 0)
        assert np.array_equal(o[:, a:b], od[0]) and np.array_equal(lse[:, a:b], ld[0])


def test_sampled_rows_match_full():
    q, k, v = (rnd((2, 3, 50, 8), s) for s in (35, 36, 37))
    idx = np.array([[0, 0, 0], [1, 2, 49], [0, 1, 17], [1, 0, 3], [0, 1, 18]])
    for mask in MASKS:
        o, lse = oracle.attention_dense(q, k, v, 0.6, mask["causal"], mask["wl"], mask["wr"])
        o_r, lse_r = oracle.attention_rows_dense(q, k, v, idx, 0.6, mask["causal"], mask["wl"],
                                                 mask["wr"])
        assert np.allclose(o_r, o[idx[:, 0], idx[:, 1], idx[:, 2]], atol=1e-13)
        assert np.allclose(lse_r, lse[idx[:, 0], idx[:, 1], idx[:, 2]], atol=1e-13)
    lens = [7, 0, 12, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qv, kv, vv = (rnd((2, cu[-1], 4), s) for s in (38, 39, 40))
    o, lse = oracle.attention_varlen(qv, kv, vv, cu, 0.6, True, 4, 0)
    idx = np.array([[0, 0], [1, 6], [0, 7], [1, 18], [1, 20], [0, 21]])
    o_r, lse_r = oracle.attention_rows_varlen(qv, kv, vv, cu, idx, 0.6, True, 4, 0)
    assert np.allclose(o_r, o[idx[:, 0], idx[:, 1]], atol=1e-13)
    assert np.allclose(lse_r, lse[idx[:, 0], idx[:, 1]], atol=1e-13)


def test_split_merge_identity():
    """Split-KV reading: attention over all keys equals the merge of attention over disjoint
    key ranges, LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s, with an empty
    range (LSE_s = -inf) contributing nothing.  Checked on the oracle, range by range."""
    q, k, v = (rnd((12, 8), s) for s in (41, 42, 43))
    o_full, lse_full = oracle.attention_head(q, k, v, 0.7)
    for cuts in ([0, 5, 12], [0, 1, 2, 12], [0, 12, 12], [0, 3, 3, 9, 12]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if a == b:
                parts.append((np.zeros_like(o_full), np.full(12, -np.inf)))
            else:
                parts.append(oracle.attention_head(q, k[a:b], v[a:b], 0.7))
        lse_s = np.stack([p[1] for p in parts])
        lse = np.log(np.sum(np.exp(lse_s), axis=0))
        o = sum(np.exp(ls - lse)[:, None] * o_s for o_s, ls in parts)
        assert np.allclose(lse, lse_full, atol=1e-12)
        assert np.allclose(o, o_full, atol=1e-12)


def test_flops_formula():
    assert oracle.flops_dense(2, 32, 8192, 128, True) == 2 * 2 * 32 * 8192 ** 2 * 128
    assert oracle.flops_dense(1, 8, 4096, 512, False) == 4 * 8 * 4096 ** 2 * 512


# ---------------------------------------------------------------------------------------------
# The pins catch plausible mistakes: plant each one in a copy of the oracle's arithmetic
# ---------------------------------------------------------------------------------------------

def _planted(mistake):
    """A copy of the oracle's head function with one plausible mistake planted."""
    def head(q, k, v, scale, causal=False, wl=-1, wr=-1):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        sc = float(np.float32(scale))
        s = (q @ k.T) * (1.0 if mistake == "no_scale" else sc)
        n_q, n_k = q.shape[0], k.shape[0]
        if mistake == "window_off_by_one" and wl >= 0:
            wl = wl - 1
        if mistake == "causal_strict" and causal:
            vis = oracle.visibility(n_q, n_k, False, wl, wr) & (
                np.arange(n_k)[None, :] < np.arange(n_q)[:, None] + (n_k - n_q))
        else:
            vis = oracle.visibility(n_q, n_k, causal, wl, wr)
        s = np.where(vis, s, -np.inf)
        m = np.max(s, axis=1)
        e = np.exp(s - m[:, None])
        lse = m + np.log(e.sum(axis=1))
        if mistake == "lse_log2":
            lse = lse / math.log(2)
        p = e / e.sum(axis=1)[:, None]
        if mistake == "reversed_v_rows":
            return p @ v[::-1], lse
        return p @ v, lse
    return head


@pytest.mark.parametrize("mistake", ["no_scale", "window_off_by_one", "causal_strict",
                                     "lse_log2", "reversed_v_rows"])
def test_pins_detect_planted_mistakes(mistake):
    head = _planted(mistake)
    n, d = 12, 12
    q, k, v = rnd((n, d), 41), rnd((n, d), 42), rnd((n, d), 43)
    caught = False
    for mask in MASKS[:4]:
        vis = page_tile_mask(n, n, mask["causal"], mask["wl"], mask["wr"], 4, 4)
        o_ref, lse_ref = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.7, vis)
        o, lse = head(q, k, v, 0.7, mask["causal"], mask["wl"], mask["wr"])
        if not (np.allclose(o, o_ref, atol=1e-12) and np.allclose(lse, lse_ref, atol=1e-12)):
            caught = True
    assert caught, mistake
