"""Pins of the backward oracle (oracle/attention_bwd.py) against things other than itself:
torch's float64 autograd through its own attention routine, central finite differences of
the forward oracle, closed forms and invariants of the softmax Jacobian, and planted mistakes
that each pin must catch.  CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_49_amd import inputs

MASKS = [
    dict(causal=False, wl=-1, wr=-1),
    dict(causal=True, wl=-1, wr=-1),
    dict(causal=True, wl=3, wr=-1),
    dict(causal=False, wl=2, wr=4),
    dict(causal=False, wl=0, wr=0),
    dict(causal=False, wl=-1, wr=1),
]


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_grads(q, k, v, do, scale, mask, gqa=False):
    """dQ, dK, dV from float64 autograd through torch's scaled_dot_product_attention (CPU)
    with an explicit boolean mask.  Rows with no visible key are left out of the loss: torch's
    softmax of an all -inf row is NaN, where the definition has P = 0."""
    nq, nk = q.shape[-2], k.shape[-2]
    vis = oracle.visibility(nq, nk, mask["causal"], mask["wl"], mask["wr"])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(vis), scale=float(np.float32(scale)),
        enable_gqa=gqa)
    keep = torch.from_numpy(vis.any(axis=1))[:, None]
    loss = torch.where(keep, o * torch.from_numpy(do), torch.zeros(())).sum()
    loss.backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("nq,nk,d", [(9, 9, 4), (16, 16, 8), (7, 12, 5), (12, 7, 3)])
def test_backward_matches_torch_autograd(mask, nq, nk, d):
    q, k, v, do = rnd((nq, d), 1), rnd((nk, d), 2), rnd((nk, d), 3), rnd((nq, d), 4)
    dq, dk, dv = oracle.attention_head_backward(q, k, v, do, 0.4, mask["causal"], mask["wl"],
                                                mask["wr"])
    tq, tk, tv = torch_grads(q, k, v, do, 0.4, mask)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(a, b, atol=1e-12, rtol=0)


@pytest.mark.parametrize("mask", MASKS[:4])
@pytest.mark.parametrize("nh,nkv", [(4, 2), (6, 1), (3, 3)])
def test_backward_gqa_matches_torch_autograd(mask, nh, nkv):
    n, d = 11, 6
    q, do = rnd((2, nh, n, d), 5), rnd((2, nh, n, d), 6)
    k, v = rnd((2, nkv, n, d), 7), rnd((2, nkv, n, d), 8)
    dq, dk, dv = oracle.attention_backward_dense(q, k, v, do, 0.3, mask["causal"], mask["wl"],
                                                 mask["wr"])
    tq, tk, tv = torch_grads(q, k, v, do, 0.3, mask, gqa=True)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(a, b, atol=1e-12, rtol=0)


@pytest.mark.parametrize("mask", MASKS[:4])
def test_backward_matches_finite_differences_of_forward(mask):
    """Central differences of L = sum(O * dO) through the forward oracle (an independent code
    path: it never forms dS), on every input element."""
    n, d, scale = 6, 3, 0.7
    q, k, v, do = rnd((n, d), 9), rnd((n, d), 10), rnd((n, d), 11), rnd((n, d), 12)
    dq, dk, dv = oracle.attention_head_backward(q, k, v, do, scale, mask["causal"], mask["wl"],
                                                mask["wr"])

    def loss(q_, k_, v_):
        o, _ = oracle.attention_head(q_, k_, v_, scale, mask["causal"], mask["wl"], mask["wr"])
        return float(np.sum(o * do))

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in np.ndindex(n, d):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            dn = loss(*args)
            assert abs((up - dn) / (2 * h) - grad[idx]) < 1e-7, (which, idx)


@pytest.mark.parametrize("mask", MASKS)
def test_backward_invariants(mask):
    """Softmax is unchanged by adding one vector to every key, so the dK rows sum to zero; the
    P rows sum to one, so the dV rows sum to the dO rows of the queries that see any key."""
    n, d = 14, 5
    q, k, v, do = rnd((n, d), 13), rnd((n, d), 14), rnd((n, d), 15), rnd((n, d), 16)
    _, dk, dv = oracle.attention_head_backward(q, k, v, do, 0.5, mask["causal"], mask["wl"],
                                               mask["wr"])
    assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    seen = oracle.visibility(n, n, mask["causal"], mask["wl"], mask["wr"]).any(axis=1)
    assert np.allclose(dv.sum(axis=0), do[seen].sum(axis=0), atol=1e-12)


def test_backward_zero_upstream_and_empty_rows():
    q, k, v = rnd((8, 4), 17), rnd((5, 4), 18), rnd((5, 4), 19)
    zero = np.zeros((8, 4))
    for g in oracle.attention_head_backward(q, k, v, zero, 0.5, True):
        assert np.array_equal(g, np.zeros_like(g))
    # bottom-right causal with Nq > Nk: the first Nq - Nk query rows see no key (zero
    # gradient); row 3 sees one key (dS = 0, so also zero); later rows see several
    do = rnd((8, 4), 20)
    dq, _, _ = oracle.attention_head_backward(q, k, v, do, 0.5, True)
    assert np.array_equal(dq[:4], np.zeros((4, 4))) and np.all(np.abs(dq[4:]).sum(axis=1) > 0)


def test_backward_one_visible_key_has_no_score_gradient():
    """A row that sees exactly one key has P = 1 there: dS = 0, so dQ = 0 and that key's
    dV is dO (window 0/0: every query sees only its own key)."""
    q, k, v, do = rnd((6, 3), 21), rnd((6, 3), 22), rnd((6, 3), 23), rnd((6, 3), 24)
    dq, dk, dv = oracle.attention_head_backward(q, k, v, do, 0.9, False, 0, 0)
    assert np.array_equal(dq, np.zeros_like(dq)) and np.array_equal(dk, np.zeros_like(dk))
    assert np.allclose(dv, do, atol=1e-15)


def test_backward_varlen_equals_per_sequence_dense():
    lens = [5, 0, 9, 1]
    q, k, v, cu = inputs.make_varlen(4, 0, 0, 4, 8, "bf16", seed=25, lengths=lens, heads_kv=2)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(26))
    qf, kf, vf, dof = (x.double().numpy() for x in (q, k, v, do))
    cu = cu.numpy()
    dq, dk, dv = oracle.attention_backward_varlen(qf, kf, vf, dof, cu, 0.3, True, 4, 0)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        gq, gk, gv = oracle.attention_backward_dense(qf[None, :, a:b], kf[None, :, a:b],
                                                     vf[None, :, a:b], dof[None, :, a:b], 0.3,
                                                     True, 4, 0)
        assert np.array_equal(dq[:, a:b], gq[0]) and np.array_equal(dk[:, a:b], gk[0])
        assert np.array_equal(dv[:, a:b], gv[0])


def test_dpsum_identity():
    """The row sum of P * dP equals dO . O (O from the forward oracle)."""
    n, d = 10, 4
    q, k, v, do = rnd((n, d), 27), rnd((n, d), 28), rnd((n, d), 29), rnd((n, d), 30)
    o, lse = oracle.attention_head(q, k, v, 0.6, True)
    s = 0.6 * (q @ k.T)
    p = np.where(oracle.visibility(n, n, True), np.exp(s - lse[:, None]), 0.0)
    assert np.allclose(np.sum(p * (do @ v.T), axis=1), np.sum(do * o, axis=1), atol=1e-12)


def test_flops_backward():
    assert oracle.flops_backward_dense(2, 32, 8192, 128, True) == 2.5 * oracle.flops_dense(
        2, 32, 8192, 128, True)


def _planted_backward(mistake):
    def head(q, k, v, do, scale, causal=False, wl=-1, wr=-1):
        sc = float(np.float32(scale))
        vis = oracle.visibility(q.shape[0], k.shape[0], causal, wl, wr)
        s = np.where(vis, sc * (q @ k.T), -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        dv = p.T @ do
        dp = do @ v.T
        dpsum = np.sum(p * dp, axis=1)
        if mistake == "no_dpsum":
            dpsum = 0 * dpsum
        ds = p * (dp - dpsum[:, None])
        if mistake == "dpsum_by_column":
            ds = p * (dp - np.sum(p * dp, axis=0)[None, :])
        dq = sc * (ds @ k)
        dk = (1.0 if mistake == "dk_unscaled" else sc) * (ds.T @ q)
        if mistake == "dv_untransposed":
            dv = p @ do
        return dq, dk, dv
    return head


@pytest.mark.parametrize("mistake", ["no_dpsum", "dpsum_by_column", "dk_unscaled",
                                     "dv_untransposed"])
def test_backward_pins_detect_planted_mistakes(mistake):
    head = _planted_backward(mistake)
    n, d = 9, 4
    q, k, v, do = rnd((n, d), 31), rnd((n, d), 32), rnd((n, d), 33), rnd((n, d), 34)
    caught = False
    for mask in MASKS[:3]:
        got = head(q, k, v, do, 0.5, mask["causal"], mask["wl"], mask["wr"])
        ref = torch_grads(q, k, v, do, 0.5, mask)
        if not all(np.allclose(a, b, atol=1e-10) for a, b in zip(got, ref)):
            caught = True
    assert caught, mistake
