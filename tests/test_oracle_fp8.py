"""Pins of the FP8 oracle (oracle/attention_fp8.py): the E4M3 decode against torch's own
float8_e4m3fn conversion for every code and against hand-worked codes, and the descale wiring
against what the definition fixes (Q/K descales act as a softmax-scale factor, the V descale
scales O and leaves the LSE alone).  CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle.attention_fp8 as fp8
from oracle import attention_dense


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0), (0x38, 1.0), (0xB8, -1.0), (0x3C, 1.5), (0x40, 2.0),
    (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x7E, 448.0),
    (0xFE, -448.0), (0x30, 0.5), (0x31, 0.5625),
])
def test_decode_hand_worked_codes(code, value):
    assert fp8.decode_e4m3(np.array([code]))[0] == value


def test_decode_nan_codes():
    assert np.isnan(fp8.decode_e4m3(np.array([0x7F, 0xFF]))).all()
    assert fp8.E4M3_MAX == fp8.decode_e4m3(np.array([0x7E]))[0]


def _codes(shape, seed):
    """Random finite E4M3 codes of moderate magnitude (|x| <= 8)."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    e = (c >> 3) & 0xF
    return np.where(e > 9, c & 0b1_0100_111, c).astype(np.uint8)  # cap the exponent field


@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (True, -1, -1), (False, 3, 2)])
def test_descale_wiring(causal, wl, wr):
    q8, k8, v8 = _codes((1, 2, 11, 8), 1), _codes((1, 2, 11, 8), 2), _codes((1, 2, 11, 8), 3)
    o1, l1 = fp8.attention_fp8_dense(q8, k8, v8, 0.25, None, None, None, causal, wl, wr)
    q, k, v = (fp8.decode_e4m3(x) for x in (q8, k8, v8))
    o0, l0 = attention_dense(q, k, v, 0.25, causal, wl, wr)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    # Q and K descales multiply the scores like the softmax scale does
    o2, l2 = fp8.attention_fp8_dense(q8, k8, v8, 0.25, 0.5, 4.0, None, causal, wl, wr)
    o3, l3 = attention_dense(q, k, v, 0.5, causal, wl, wr)
    assert np.allclose(o2, o3, atol=1e-13) and np.allclose(l2, l3, atol=1e-13)
    # the V descale scales O and leaves the LSE unchanged
    o4, l4 = fp8.attention_fp8_dense(q8, k8, v8, 0.25, None, None, 0.125, causal, wl, wr)
    assert np.allclose(o4, 0.125 * o0, atol=1e-15) and np.array_equal(l4, l0)


def test_varlen_fp8_is_varlen_of_decoded():
    q8, k8, v8 = _codes((2, 20, 4), 4), _codes((1, 20, 4), 5), _codes((1, 20, 4), 6)
    cu = np.array([0, 7, 7, 20])
    o, l = fp8.attention_fp8_varlen(q8, k8, v8, cu, 0.3, 2.0, 0.5, 3.0, True, 5, 0)
    from oracle import attention_varlen
    q, k, v = fp8.decode_e4m3(q8) * 2.0, fp8.decode_e4m3(k8) * 0.5, fp8.decode_e4m3(v8) * 3.0
    o0, l0 = attention_varlen(q, k, v, cu, 0.3, True, 5, 0)
    assert np.array_equal(o, o0) and np.array_equal(l, l0)
    assert math.isfinite(float(np.max(np.abs(o))))
