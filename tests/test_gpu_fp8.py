"""GPU parity of the FP8 forward (through the C ABI, head dims 64/128/256) against the fp64
CPU oracle, which attends over the dequantized tensors (code * descale).

Bars.  The LSE is held to the forward's bar, 1e-3 * max(1, |LSE|).  The products of E4M3
values are exact, but the FP8 MFMA's internal sums are not round-to-nearest fp32: the measured
score error grows like d * 2^-24 * |S| (8.8e-4 in the LSE of the sharp d = 256 case, where |S|
reaches about 50), so no tighter bar holds.  O carries the rounding of P to E4M3 before the P V product: a
relative error of at most 2^-4 for P in the normal range and 2^-10 absolute below it, with P
scaled so that its row sum is at least 256.  Per element that bounds
    |O_gpu - O_ref| <= 2^-4 * (P|V|)_i + 2^-18 * sum_{j visible} |V_j| + 2^-8 |O_ref| + 1e-6,
where P|V| is the attention of |V| (computed by the oracle) and 2^-8 covers the bf16 output.
A sharp-softmax case, where O is close to one V row, catches key-order mistakes that the bound
alone could hide; 24 seeded random configurations (head dim, grouped heads, batch, length, mask
mode, output dtype) cover combinations the listed cases do not."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention_fp8 as ofp8
from exact_attention_49_amd import attn_fwd_fp8, attn_fwd_varlen_fp8, inputs
from tests.gpu_helpers import to64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MASKS = {
    "none": dict(causal=False, wl=-1, wr=-1),
    "causal": dict(causal=True, wl=-1, wr=-1),
    "window_40_0": dict(causal=True, wl=40, wr=0),
    "window_30_70": dict(causal=False, wl=30, wr=70),
}


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _quantized(shape, kv_shape, seed, value_scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    xs = [torch.randn(sh, generator=g) * value_scale for sh in (shape, kv_shape, kv_shape)]
    return [inputs.quantize_fp8(x) for x in xs]


def _codes(t):
    return t.view(torch.uint8).numpy()


def _check(o, lse, o_ref, lse_ref, bound, what):
    o, lse = to64(o), to64(lse)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    err = np.abs(o - o_ref)
    assert np.all(err <= bound), f"{what}: O err {float(np.max(err / bound)):.2f} x bound"
    fin = np.isfinite(lse_ref)
    assert np.all(lse[~fin] == -np.inf)
    d = np.abs(lse[fin] - lse_ref[fin])
    assert np.all(d <= 1e-3 * np.maximum(1.0, np.abs(lse_ref[fin]))), f"{what}: LSE {d.max():.2e}"
    return float(np.max(err / bound))


def _dense_case(bsz, hq, hkv, n, m, seed, value_scale=1.0, out_dtype=torch.bfloat16, d=128):
    (q8, dq), (k8, dk), (v8, dv) = _quantized((bsz, hq, n, d), (bsz, hkv, n, d), seed,
                                              value_scale)
    dts = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in (dq, dk, dv)]
    o, lse = attn_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), *dts, causal=m["causal"],
                          window_left=m["wl"], window_right=m["wr"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = ofp8.attention_fp8_dense(_codes(q8), _codes(k8), _codes(v8), scale, dq, dk,
                                              dv, m["causal"], m["wl"], m["wr"])
    vabs = np.abs(ofp8.decode_e4m3(_codes(v8))) * float(np.float32(dv))
    qd = ofp8.decode_e4m3(_codes(q8)) * float(np.float32(dq))
    kd = ofp8.decode_e4m3(_codes(k8)) * float(np.float32(dk))
    a, _ = oracle.attention_dense(qd, kd, vabs, scale, m["causal"], m["wl"], m["wr"])
    vis = oracle.visibility(n, n, m["causal"], m["wl"], m["wr"]).astype(np.float64)
    g = hq // hkv
    s = np.stack([np.stack([vis @ vabs[b, h // g] for h in range(hq)]) for b in range(bsz)])
    bound = 2.0 ** -4 * a + 2.0 ** -18 * s + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    return _check(o, lse, o_ref, lse_ref, bound, f"fp8 {bsz}x{hq}/{hkv}x{n} {m}")


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("n", [1, 63, 300, 1025])
def test_fp8_dense(mask, n):
    _announce(f"fp8 dense n={n} {mask}")
    _dense_case(2, 2, 2, n, MASKS[mask], seed=3100 + n)


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("d", [64, 256])
def test_fp8_other_head_dims(d, mask):
    _announce(f"fp8 d={d} {mask}")
    _dense_case(2, 2, 2, 300, MASKS[mask], seed=3150 + d, d=d)
    _dense_case(1, 2, 2, 1025, MASKS[mask], seed=3160 + d, d=d)


@pytest.mark.parametrize("d", [64, 256])
def test_fp8_other_head_dims_gqa_and_sharp(d):
    _announce(f"fp8 d={d} gqa, sharp")
    _dense_case(1, 6, 2, 257, MASKS["causal"], seed=3170 + d, d=d)
    _dense_case(1, 2, 2, 400, MASKS["causal"], seed=3180 + d, value_scale=4.0, d=d)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (6, 1)])
def test_fp8_gqa(hq, hkv):
    _announce(f"fp8 gqa {hq}/{hkv}")
    _dense_case(1, hq, hkv, 500, MASKS["causal"], seed=3200 + hq)


def test_fp8_fp16_output():
    _announce("fp8 fp16 out")
    _dense_case(1, 2, 2, 257, MASKS["causal"], seed=3300, out_dtype=torch.float16)


def test_fp8_sharp_softmax_picks_the_right_rows():
    """Q and K scaled up: each row's softmax is nearly one-hot, so O is close to a single V row
    and any mix-up of key order between P and V shows as an error of order |V|."""
    _announce("fp8 sharp")
    _dense_case(1, 2, 2, 400, MASKS["causal"], seed=3400, value_scale=4.0)


def test_fp8_big_grid():
    _announce("fp8 big grid")
    _dense_case(2, 16, 4, 2048, MASKS["causal"], seed=3500)


def test_fp8_descale_none_means_one():
    _announce("fp8 no descales")
    g = torch.Generator("cpu").manual_seed(3600)
    q8, k8, v8 = ((torch.randn(1, 2, 130, 128, generator=g)).to(torch.float8_e4m3fn)
                  for _ in range(3))
    o, lse = attn_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = ofp8.attention_fp8_dense(_codes(q8), _codes(k8), _codes(v8),
                                              1 / math.sqrt(128), causal=True)
    assert float(np.max(np.abs(to64(o) - o_ref))) <= 0.1
    assert float(np.max(np.abs(to64(lse) - lse_ref))) <= 1e-3


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mask", ["causal", "window_30_70"])
def test_fp8_varlen(mask, d):
    _announce(f"fp8 varlen d={d} {mask}")
    m = MASKS[mask]
    lens = [1, 0, 64, 300, 129, 3]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    total = int(cu[-1])
    (q8, dq), (k8, dk), (v8, dv) = _quantized((4, total, d), (2, total, d), 3700 + d)
    dts = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in (dq, dk, dv)]
    o, lse = attn_fwd_varlen_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), cu.to(DEV), max(lens),
                                 *dts, causal=m["causal"], window_left=m["wl"],
                                 window_right=m["wr"])
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    cun = cu.numpy()
    o_ref, lse_ref = ofp8.attention_fp8_varlen(_codes(q8), _codes(k8), _codes(v8), cun, scale,
                                               dq, dk, dv, m["causal"], m["wl"], m["wr"])
    qd = ofp8.decode_e4m3(_codes(q8)) * float(np.float32(dq))
    kd = ofp8.decode_e4m3(_codes(k8)) * float(np.float32(dk))
    vabs = np.abs(ofp8.decode_e4m3(_codes(v8))) * float(np.float32(dv))
    a, _ = oracle.attention_varlen(qd, kd, vabs, cun, scale, m["causal"], m["wl"], m["wr"])
    s = np.zeros_like(a)
    for i in range(len(lens)):
        lo, hi = cun[i], cun[i + 1]
        if hi > lo:
            vis = oracle.visibility(hi - lo, hi - lo, m["causal"], m["wl"], m["wr"]).astype(float)
            for h in range(4):
                s[h, lo:hi] = vis @ vabs[h // 2, lo:hi]
    bound = 2.0 ** -4 * a + 2.0 ** -18 * s + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    _check(o, lse, o_ref, lse_ref, bound, f"fp8 varlen {mask}")


def test_workload_fp8_causal_d128_n8192_full():
    """The FP8 workload at full size: every row of every head against the oracle, each element
    against the error bound above."""
    from concurrent.futures import ThreadPoolExecutor
    from tests.gpu_helpers import _oracle_workers
    w = inputs.WORKLOADS["fp8_causal_d128_n8192"]
    _announce(w.name)
    (q8, dq), (k8, dk), (v8, dv) = (inputs.quantize_fp8(x) for x in inputs.make_workload(w))
    dts = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in (dq, dk, dv)]
    o, lse = attn_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), *dts, causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    qd = ofp8.decode_e4m3(_codes(q8)) * float(np.float32(dq))
    kd = ofp8.decode_e4m3(_codes(k8)) * float(np.float32(dk))
    vd = ofp8.decode_e4m3(_codes(v8)) * float(np.float32(dv))
    heads = [(b, h) for b in range(2) for h in range(32)]

    def one(bh):
        b, h = bh
        o_ref, lse_ref = oracle.attention_head(qd[b, h], kd[b, h], vd[b, h], w.softmax_scale,
                                               True)
        a, _ = oracle.attention_head(qd[b, h], kd[b, h], np.abs(vd[b, h]), w.softmax_scale,
                                     True)
        s = np.cumsum(np.abs(vd[b, h]), axis=0)   # causal row r sees keys 0..r
        bound = 2.0 ** -4 * a + 2.0 ** -18 * s + 2.0 ** -8 * np.abs(o_ref) + 1e-6
        return _check(o[b, h], lse[b, h], o_ref, lse_ref, bound, f"{w.name} b={b} h={h}")

    with ThreadPoolExecutor(_oracle_workers()) as ex:
        worst = max(ex.map(one, heads))
    assert worst <= 1.0


def _draw_fp8(i):
    rng = np.random.default_rng(40260 + i)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.integers(1, 4))
    hq = hkv * int(rng.choice([1, 2, 4]))
    mode = int(rng.integers(0, 4))
    causal, wl, wr = [(False, -1, -1), (True, -1, -1),
                      (True, int(rng.integers(0, 300)), -1),
                      (False, int(rng.integers(0, 200)), int(rng.integers(0, 200)))][mode]
    out = torch.bfloat16 if bool(rng.integers(0, 2)) else torch.float16
    return d, hq, hkv, int(rng.integers(1, 3)), int(rng.integers(1, 700)), \
        dict(causal=causal, wl=wl, wr=wr), out


@pytest.mark.parametrize("i", range(24))
def test_fp8_random_configuration(i):
    # seeded random head dim, grouped heads, batch, length, mask mode and output dtype, against
    # the bound above
    d, hq, hkv, b, n, m, out = _draw_fp8(i)
    _announce(f"fp8 random {i}: d={d} B{b} H{hq}/{hkv} N{n} {m} {out}")
    _dense_case(b, hq, hkv, n, m, seed=4100 + i, out_dtype=out, d=d)
