"""Benchmark of the exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

With no --workload, the headline workload (B=2 H=32 N=8192 d=128 bf16 causal) is timed and its
JSON line also carries `configs`: the same measurement for all five synthetic configurations
(TFLOP/s, % of the MFMA peak, per-launch time, algorithmic and counter-measured HBM figures,
MFMA busy fraction from the committed counters, the oracle's rate on the host cores and the
parity of the GPU's outputs against the oracle on the units it computed).

One step = one forward pass (one attn_fwd / attn_fwd_varlen call, attn_fwd_gqa for the
grouped-query workload; for the split-KV workload one attn_fwd_splitkv call, which runs the
split sweep and the merge; for the backward workload one attn_bwd call, its two kernels, with
the forward's O and LSE computed before timing) over the workload's
inputs, which are resident in HBM before timing starts.  The step first repeats untimed for
0.3 s while the engine clock ramps up under load (config.clock_settle records how many), then
W untimed warm-up steps, then exactly K timed steps between two device synchronisations.
Rank 0 prints one JSON line:

  value    whole-job TFLOP/s with F = 4*B*H*N^2*d, halved when causal (packed batches count
           the visible (query, key) pairs: F = 4*H*d*sum_s pairs_s)
  roofline the dominant (only) kernel against MI355X's dense fp16/bf16 MFMA peak, from the
           per-launch durations measured with HIP events on the launch stream
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same workload, with the
           GPU's outputs compared to the oracle's on that sample (parity)

Besides the warm timing, a short second pass times the same launches with 512 MiB of other
device traffic between them (reported as cold_cache; --no-cold skips it).  Other flags:
--flush makes the main timing cache-cold too, --list-workloads, --calibrate-copy runs only a
plain device copy of known size (for scaling HBM counters).
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d, halved if causal) and % of MFMA peak"
METRIC_BWD = ("attention bwd TFLOP/s (2.5·4·B·H·N²·d, halved if causal) and % of MFMA peak")
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6,    # MI355X dense MFMA, AMD's published figures
               "fp8": 5033.2}
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "causal_bf16_d128_n8192"
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


# The sources that build each kernel family: its device code, the shared device helpers and
# the host code that sizes and dispatches its launches.
_SHARED = ("attn_common.h", "attn_api.hip")
_FWD_SHARED = _SHARED + ("attn_dispatch.h",)
KERNEL_SOURCES = {
    "pingpong": _FWD_SHARED + ("attn_fwd_pingpong.h", "attn_fwd_d128.hip"),
    "generic": _FWD_SHARED + ("attn_fwd_kernel.h", "attn_merge.h", "attn_fwd_d64.hip",
                              "attn_fwd_d128.hip"),
    "wide": _FWD_SHARED + ("attn_fwd_wide.h", "attn_merge.h", "attn_fwd_d256.hip",
                           "attn_fwd_d512.hip"),
    "fp8": _SHARED + ("attn_fwd_fp8.h", "attn_fwd_fp8.hip"),
    "bwd": _SHARED + ("attn_bwd.h", "attn_bwd_d64.hip", "attn_bwd_d128.hip"),
    "persistent": _FWD_SHARED + ("attn_fwd_pingpong.h", "attn_fwd_persistent.h",
                                 "attn_fwd_pers.hip"),
}


def kernel_family(w, cu=None) -> str:
    """The KERNEL_SOURCES family of the kernel(s) a workload's step launches."""
    if w.backward or w.fp8:
        return "bwd" if w.backward else "fp8"
    name = kernel_name(w, cu)
    if name.startswith("attn_fwd_wide_kernel"):
        return "wide"
    return "pingpong" if name == "attn_fwd_pp_kernel" else "generic"


def _code_only(text: str) -> str:
    """C++ source with its comments removed and whitespace runs collapsed (string literals in
    these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(family: str) -> str:
    """Hash of the code (comments and layout excluded) of the HIP sources of one kernel family
    (KERNEL_SOURCES): recorded HBM counters are only valid for the kernels they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_49_amd", "csrc")
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def visible_pairs(n: int, causal: bool, wl: int, wr: int) -> int:
    """Exact number of (query, key) pairs with the key visible, for one sequence (Nq = Nk)."""
    total = 0
    for i in range(n):
        lo = 0 if wl < 0 else max(0, i - wl)
        hi = n - 1
        if causal:
            hi = i
        elif wr >= 0:
            hi = min(n - 1, i + wr)
        total += hi - lo + 1
    return total


def workload_flops(w, cu=None) -> float:
    """Forward: 4*B*H*N^2*d, halved when causal (packed: 4*H*d*visible pairs).  Backward: 2.5
    times that (five N x N x d products against the forward's two)."""
    if w.backward:
        return 2.5 * workload_flops(dataclasses.replace(w, backward=False), cu)
    if w.varlen:
        lens = (cu[1:] - cu[:-1]).tolist()
        pairs = sum(visible_pairs(int(n), w.causal, w.window_left, w.window_right) for n in lens)
        return 4.0 * w.heads * w.head_dim * pairs
    f = 4.0 * w.batch * w.heads * w.seqlen ** 2 * w.head_dim
    return f / 2 if w.causal else f


def workload_bytes(w, cu=None) -> float:
    """Algorithmic HBM bytes per launch: Q, K, V read once, O written once (2 B each) and
    LSE written once (4 B per row); K and V have the key/value head count.  Backward: Q, K, V,
    O, dO read, dQ, dK, dV written (2 B each), LSE read, dPsum written and read (4 B each)."""
    tokens = int(cu[-1]) if w.varlen else w.batch * w.seqlen
    if w.fp8:  # 1-byte Q, K, V; 2-byte O
        return tokens * (w.heads * (w.head_dim * 3 + 4) + w.kv_heads * 2 * w.head_dim)
    if w.backward:
        return tokens * (w.heads * (4 * w.head_dim * 2 + 12) + w.kv_heads * 4 * w.head_dim * 2)
    return tokens * (w.heads * (2 * w.head_dim * 2 + 4) + w.kv_heads * 2 * w.head_dim * 2)


def kernel_name(w, cu=None) -> str:
    """The kernel the library launches for a workload (mirrors the host dispatch: the wide
    kernel for d >= 256, the generic kernel for d = 64, and for d = 128 the ping-pong kernel
    once the grid of 256-row tiles has at least 256 workgroups (384 under a causal or window
    mask), else the generic one)."""
    if w.backward:
        return "attn_bwd_dq_kernel + attn_bwd_dkdv_kernel (one step)"
    if w.fp8:
        return "attn_fwd_fp8_kernel"
    if w.splitkv:  # one step = the split sweep and the merge
        base = "attn_fwd_wide_kernel" if w.head_dim >= 256 else "attn_fwd_kernel"
        return f"{base} (split-KV) + attn_merge_kernel"
    if w.head_dim >= 256:
        return "attn_fwd_wide_kernel"
    if w.head_dim == 64:
        return "attn_fwd_kernel"
    if w.varlen:
        tiles = w.heads * ((int(cu[-1]) + 255) // 256)
        longest = int((cu[1:] - cu[:-1]).max())
    else:
        tiles = w.batch * w.heads * ((w.seqlen + 255) // 256)
        longest = w.seqlen
    # masked unless the windows cover every key (a window as long as the sequence is none)
    masked = (w.causal or 0 <= w.window_left < longest or 0 <= w.window_right < longest)
    return "attn_fwd_pp_kernel" if tiles >= (384 if masked else 256) else "attn_fwd_kernel"


def load_counters(w, cu=None):
    """Counter figures for a workload's kernel from the committed rocprofv3 summary
    (profiles/<workload>_hbm_traffic.txt: `key: value` lines), if it was taken on the current
    kernel sources; else None.  Keys used here: hbm_bytes_per_launch (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy's readings) and, where recorded, mfma_busy_frac and
    clock_mhz_measured (SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE)."""
    path = os.path.join(TRAFFIC_DIR, f"{w.name}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.partition(":")
            if sep and not key.startswith("#"):
                rec[key.strip()] = val.strip()
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel_family(w, cu)):
        return None
    out = {}
    for key in ("hbm_bytes_per_launch", "mfma_busy_frac", "clock_mhz_measured",
                "sq_valu_mfma_busy_cycles", "grbm_gui_active"):
        try:
            out[key] = float(rec[key])
        except (KeyError, ValueError):
            pass
    return out


def load_traffic(w, cu=None):
    """HBM bytes per launch from the committed counter summary (see load_counters), or None."""
    c = load_counters(w, cu)
    return None if c is None else c.get("hbm_bytes_per_launch")


def _cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f
                         if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover
        return None


class _Parity:
    """Element-wise comparison of the GPU's outputs with the oracle's on the units the CPU
    baseline computed (the same bars as the parity tests)."""

    def __init__(self):
        self.o_err, self.lse_err, self.rows = 0.0, 0.0, 0

    def add(self, o_gpu, lse_gpu, o_ref, lse_ref):
        import numpy as np
        o_gpu = o_gpu.double().numpy()
        self.o_err = max(self.o_err, float(np.max(np.abs(o_gpu - o_ref))))
        lse_gpu = lse_gpu.double().numpy()
        fin = np.isfinite(lse_ref)
        if fin.any():
            rel = np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
            self.lse_err = max(self.lse_err, float(np.max(rel)))
        self.rows += int(o_ref.shape[0])

    def record(self, dtype):
        return {"max_abs_err_O": self.o_err, "bar_O": 2e-2 if dtype == "bf16" else 5e-3,
                "lse_rel_err": self.lse_err, "bar_lse_rel": 1e-3, "rows_compared": self.rows}


def cpu_baseline(w, q, k, v, cu, budget_s: float = 20.0, o_gpu=None, lse_gpu=None):
    """Time the fp64 oracle on a bounded sample: whole (batch, head) pairs, or whole
    (sequence, head) pairs for a packed batch, until the budget is spent.  With the GPU's
    outputs (CPU tensors) given, the oracle's results on the sampled units are also compared
    with them (recorded as `parity`)."""
    import oracle
    threads = _cpu_threads()
    par = _Parity() if o_gpu is not None else None
    done_flops, t_total, units = 0.0, 0.0, []
    if w.varlen:
        cu_l = cu.tolist()
        order = [(h, s) for s in range(w.num_seqs) for h in range(w.heads)]
        g = w.heads // w.kv_heads
        for (h, s) in order:
            a, b = cu_l[s], cu_l[s + 1]
            qs = q[h, a:b].float().numpy()
            ks, vs = (x[h // g, a:b].float().numpy() for x in (k, v))
            t0 = time.perf_counter()
            o_ref, lse_ref = oracle.attention_head(qs, ks, vs, w.softmax_scale, w.causal,
                                                   w.window_left, w.window_right)
            t_total += time.perf_counter() - t0
            if par is not None:
                par.add(o_gpu[h, a:b], lse_gpu[h, a:b], o_ref, lse_ref)
            done_flops += 4.0 * w.head_dim * visible_pairs(b - a, w.causal, w.window_left,
                                                           w.window_right)
            units.append(f"seq{s}/h{h}")
            if t_total >= budget_s:
                break
        sample = (f"{len(units)} of {len(order)} (sequence, head) pairs of the packed batch, "
                  "whole, fp64 numpy")
    elif w.backward:
        f_head = 10.0 * w.seqlen ** 2 * w.head_dim / (2 if w.causal else 1)
        g = w.heads // w.kv_heads
        do = inputs_upstream(w, q)
        for b in range(w.batch):
            for h in range(w.heads):
                qs, dos = q[b, h].float().numpy(), do[b, h].float().numpy()
                ks, vs = (x[b, h // g].float().numpy() for x in (k, v))
                t0 = time.perf_counter()
                oracle.attention_head_backward(qs, ks, vs, dos, w.softmax_scale, w.causal,
                                               w.window_left, w.window_right)
                t_total += time.perf_counter() - t0
                done_flops += f_head
                units.append((b, h))
                if t_total >= budget_s:
                    break
            if t_total >= budget_s:
                break
        sample = (f"{len(units)} of {w.batch * w.heads} (batch, head) pairs, whole backward "
                  f"(N={w.seqlen}, d={w.head_dim}), fp64 numpy")
    else:
        f_head = 4.0 * w.seqlen ** 2 * w.head_dim / (2 if w.causal else 1)
        g = w.heads // w.kv_heads
        for b in range(w.batch):
            for h in range(w.heads):
                qs = q[b, h].float().numpy()
                ks, vs = (x[b, h // g].float().numpy() for x in (k, v))
                t0 = time.perf_counter()
                o_ref, lse_ref = oracle.attention_head(qs, ks, vs, w.softmax_scale, w.causal,
                                                       w.window_left, w.window_right)
                t_total += time.perf_counter() - t0
                if par is not None:
                    par.add(o_gpu[b, h], lse_gpu[b, h], o_ref, lse_ref)
                done_flops += f_head
                units.append((b, h))
                if t_total >= budget_s:
                    break
            if t_total >= budget_s:
                break
        sample = (f"{len(units)} of {w.batch * w.heads} (batch, head) pairs, whole "
                  f"(N={w.seqlen}, d={w.head_dim}), fp64 numpy")
    out = {"value": done_flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle", "sample": sample, "seconds": round(t_total, 2),
           "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}
    if par is not None:
        out["parity"] = par.record(w.dtype)
    return out


def inputs_upstream(w, q):
    """The workload's upstream gradient dO (a seeded draw, like the inputs)."""
    from exact_attention_49_amd import inputs
    return inputs.make_upstream(q.shape, w.dtype, seed=w.seed + 100, value_scale=w.value_scale)


def inputs_dequantized(codes, descale):
    """What E4M3 codes stand for (code * descale), as float32 CPU tensors for the oracle."""
    return codes.float() * float(descale)


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 5) -> None:
    import torch
    dev = torch.device("cuda:0")
    x = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps}))


# The five synthetic configurations the benchmark reports (the headline is the long causal
# one); each is also a parity workload of the tests.
FIVE_CONFIGS = ("tiny_fp16_d64", "causal_bf16_d128_n2048", "causal_bf16_d128_n8192",
                "varlen_bf16_d64_w1024", "dense_fp16_d512_n4096")


def run_workload(w, steps: int, warmup: int, flush: bool = False, cold: bool = True,
                 cpu_budget: float | None = 20.0, settle_s: float = 0.3) -> dict:
    """Time `steps` steps of one workload after `warmup` untimed ones and return its record:
    whole-job throughput, the dominant kernel's roofline from HIP-event launch durations,
    counter figures from profiles/ (when taken on the current sources), and, unless
    cpu_budget is None, the CPU oracle's rate on a bounded sample with the GPU's outputs
    compared to it there."""
    import torch

    from exact_attention_49_amd import (attn_bwd, attn_fwd, attn_fwd_fp8, attn_fwd_gqa,
                                        attn_fwd_splitkv, attn_fwd_varlen, attn_fwd_varlen_gqa,
                                        bwd_workspace_size, inputs, splitkv_num_splits,
                                        splitkv_workspace_size, varlen_bwd_workspace_size)
    dev = torch.device("cuda:0")
    cu = None
    if w.varlen:
        q, k, v, cu = inputs.make_workload(w)
        max_len = int((cu[1:] - cu[:-1]).max())
    else:
        q, k, v = inputs.make_workload(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    lse_shape = (w.heads, qd.shape[1]) if w.varlen else (w.batch, w.heads, w.seqlen)
    lsed = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    cud = cu.to(dev) if cu is not None else None
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if flush else None

    ws = None
    if w.splitkv:  # caller-owned workspace, allocated before any timing
        nbytes = splitkv_workspace_size(w.batch, w.heads, w.seqlen, w.head_dim, 0, w.causal,
                                        w.window_left)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if w.fp8:  # E4M3 inputs with per-tensor descales, quantised before timing
        (q8, dsq), (k8, dsk), (v8, dsv) = (inputs.quantize_fp8(x) for x in (q, k, v))
        qd, kd, vd = q8.to(dev), k8.to(dev), v8.to(dev)
        descales = [torch.tensor([x], dtype=torch.float32, device=dev) for x in (dsq, dsk, dsv)]
        od = torch.empty(q.shape, dtype=w.torch_dtype, device=dev)
        q, k, v = (inputs_dequantized(x, s) for x, s in ((q8, dsq), (k8, dsk), (v8, dsv)))
    if w.backward:  # the forward's outputs, dO, gradient buffers and workspace, before timing
        attn_fwd_gqa(qd, kd, vd, causal=w.causal, window_left=w.window_left,
                     window_right=w.window_right, out=od, lse=lsed)
        dod = inputs_upstream(w, q).to(dev)
        dqd, dkd, dvd = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        nbytes = (varlen_bwd_workspace_size(int(cu[-1]), w.heads) if w.varlen
                  else bwd_workspace_size(w.batch, w.heads, w.seqlen))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step():
        if w.fp8:
            attn_fwd_fp8(qd, kd, vd, *descales, causal=w.causal, window_left=w.window_left,
                         window_right=w.window_right, out_dtype=w.torch_dtype, out=od,
                         lse=lsed)
        elif w.backward:
            attn_bwd(qd, kd, vd, od, lsed, dod, causal=w.causal, window_left=w.window_left,
                     window_right=w.window_right, dq=dqd, dk=dkd, dv=dvd, workspace=ws)
        elif w.splitkv:
            attn_fwd_splitkv(qd, kd, vd, causal=w.causal, window_left=w.window_left,
                             window_right=w.window_right, out=od, lse=lsed, num_splits=0,
                             workspace=ws)
        elif w.varlen:
            (attn_fwd_varlen_gqa if w.heads_kv else attn_fwd_varlen)(
                qd, kd, vd, cud, max_len, causal=w.causal, window_left=w.window_left,
                window_right=w.window_right, out=od, lse=lsed)
        else:
            (attn_fwd_gqa if w.heads_kv else attn_fwd)(
                qd, kd, vd, causal=w.causal, window_left=w.window_left,
                window_right=w.window_right, out=od, lse=lsed)

    # The engine clock ramps up over the first 0.1-0.2 s of sustained load: repeat the step for
    # settle_s seconds first, so that the warm-up and the timed steps run at the steady clock.
    settle_steps = 0
    torch.cuda.synchronize()
    t_settle = time.perf_counter() + settle_s
    while time.perf_counter() < t_settle:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
        settle_steps += 4
    for _ in range(warmup):
        if flush_buf is not None:
            flush_buf.fill_(1)
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)   # the stream the kernels are launched on

    def timed(n, flush_with):
        """Launch n steps; returns (wall seconds, per-launch ms from HIP events)."""
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            if flush_with is not None:
                flush_with.fill_(1)
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, [a.elapsed_time(b) for a, b in zip(starts, ends)]

    wall, launch_ms = timed(steps, flush_buf)
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    ms_per_step = wall / steps * 1e3
    srt = sorted(launch_ms)
    med_launch_ms, min_launch_ms = srt[len(srt) // 2], srt[0]
    # the same launches with 512 MiB of other traffic between them (cold caches), for context
    cold_rec = None
    if cold:
        cold_buf = flush_buf if flush_buf is not None else torch.empty(
            512 << 20, dtype=torch.uint8, device=dev)
        _, cold_ms = timed(min(steps, 20), cold_buf)
        cold_avg = sum(cold_ms) / len(cold_ms)
        cold_rec = {"avg_launch_ms": round(cold_avg, 4),
                    "tflops": round(workload_flops(w, cu) / (cold_avg / 1e3) / 1e12, 2),
                    "launches": len(cold_ms), "between_launches": "512 MiB device fill"}
        del cold_buf

    flops = workload_flops(w, cu)
    algo_bytes = workload_bytes(w, cu)
    # the device as the HIP runtime reports it: the published peak assumes 256 CUs at 2.4 GHz
    # and 4096 dense 16-bit MFMA flops per clock per CU (twice that for FP8)
    from exact_attention_49_amd.binding import device_info
    dev_info = device_info(0)
    clock_peak = (dev_info["compute_units"] * dev_info["clock_mhz"] * 1e6
                  * (8192 if w.fp8 else 4096) / 1e12)
    value = flops * steps / wall / 1e12
    achieved = flops / avg_launch_s / 1e12
    peak = PEAK_TFLOPS["fp8" if w.fp8 else w.dtype]
    counters = load_counters(w, cu) or {}
    traffic = counters.get("hbm_bytes_per_launch")

    config = {"workload": w.name, "heads": w.heads, "heads_kv": w.kv_heads,
              "head_dim": w.head_dim, "dtype": w.dtype,
              "causal": w.causal, "window_left": w.window_left,
              "window_right": w.window_right, "seed": w.seed, "value_scale": w.value_scale}
    # untimed launches before the warm-up steps while the engine clock settles
    config["clock_settle"] = {"seconds": settle_s, "steps": settle_steps}
    if w.varlen:
        lens = (cu[1:] - cu[:-1]).tolist()
        config.update(num_seqs=w.num_seqs, total_tokens=int(cu[-1]), lengths=lens,
                      flops_counted="4*H*d*(visible pairs)",
                      flops_formula_literal=sum(2.0 * w.heads * n * n * w.head_dim
                                                for n in lens))
    else:
        config.update(batch=w.batch, seqlen=w.seqlen)
    if w.backward:
        config.update(entry_point="attn_bwd", direction="backward (dQ, dK, dV)",
                      flops_counted="2.5 x forward (five N x N x d products)")
    if w.splitkv:
        config.update(entry_point="attn_fwd_splitkv",
                      num_splits=splitkv_num_splits(w.batch, w.heads, w.seqlen, w.head_dim,
                                                    w.causal, w.window_left))
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": traffic, "kernel": kernel_name(w, cu),
            "avg_launch_ms": round(avg_launch_s * 1e3, 4),
            "median_launch_ms": round(med_launch_ms, 4),
            "min_launch_ms": round(min_launch_ms, 4),
            "algorithmic_bytes": algo_bytes,
            "algorithmic_hbm_gbs": round(algo_bytes / avg_launch_s / 1e9, 1)}
    if traffic is not None:
        roof["traffic_over_algorithmic"] = round(traffic / algo_bytes, 3)
        roof["measured_hbm_gbs"] = round(traffic / avg_launch_s / 1e9, 1)
    if "mfma_busy_frac" in counters:
        # SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCDs), from the profile
        roof["mfma_busy_frac"] = counters["mfma_busy_frac"]
        roof["mfma_busy_normalisation"] = ("SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x "
                                           "GRBM_GUI_ACTIVE / 8 XCDs)")
    if "clock_mhz_measured" in counters:
        roof["clock_mhz_measured"] = counters["clock_mhz_measured"]
    if "sq_valu_mfma_busy_cycles" in counters:
        # the profile's MFMA-busy cycles per dispatch against this run's launch time at the
        # nominal clock (equal to frac when the MFMA count is the algorithmic one)
        roof["mfma_busy_frac_nominal"] = round(
            counters["sq_valu_mfma_busy_cycles"] / 1024 / (avg_launch_s * 2.4e9), 4)
    out = {
        "metric": METRIC_BWD if w.backward else METRIC, "value": round(value, 2),
        "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8" if w.fp8 else w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, no dataset)", "config": config,
        "pct_of_mfma_peak": round(100 * value / peak, 2),
        "flops_per_step": flops, "cache": "flushed 512 MiB between steps" if flush
        else "warm (back-to-back launches)",
        "roofline": roof,
        "kernel_source_hash": kernel_source_hash(kernel_family(w, cu)),
        "device": {**dev_info, "peak_tflops_at_reported_clock": round(clock_peak, 1),
                   "pct_of_clock_peak": round(100 * value / clock_peak, 2)},
    }
    if cold_rec is not None:
        out["cold_cache"] = cold_rec
    if w.splitkv:  # the same problem through the plain entry point, for context
        def plain():
            attn_fwd_gqa(qd, kd, vd, causal=w.causal, window_left=w.window_left,
                         window_right=w.window_right, out=od, lse=lsed)
        for _ in range(3):
            plain()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(20):
            plain()
        ev1.record(stream)
        torch.cuda.synchronize()
        pm = ev0.elapsed_time(ev1) / 20
        out["plain_path"] = {"entry_point": "attn_fwd_gqa", "avg_launch_ms": round(pm, 4),
                             "tflops": round(flops / (pm / 1e3) / 1e12, 2)}
    if cpu_budget is not None:
        compare = not (w.backward or w.fp8)
        o_cpu = od.cpu() if compare else None
        l_cpu = lsed.cpu() if compare else None
        del qd, kd, vd, od, lsed
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, cu, cpu_budget, o_cpu, l_cpu)
        out["cpu_baseline"]["speedup_gpu_over_cpu"] = round(
            value / out["cpu_baseline"]["value"], 1)
    return out


def config_summary(rec: dict) -> dict:
    """The per-configuration row of the default run's five-config record."""
    roof = rec["roofline"]
    row = {"workload": rec["config"]["workload"], "kernel": roof["kernel"],
           "avg_launch_us": round(roof["avg_launch_ms"] * 1e3, 2),
           "ms_per_step": rec["ms_per_step"], "steps": rec["steps"],
           "tflops": roof["achieved"], "pct_of_mfma_peak": round(100 * roof["frac"], 2),
           "tflops_wall": rec["value"],
           "algorithmic_bytes": roof["algorithmic_bytes"],
           "algorithmic_hbm_gbs": roof["algorithmic_hbm_gbs"]}
    for key in ("traffic", "traffic_over_algorithmic", "measured_hbm_gbs", "mfma_busy_frac",
                "mfma_busy_frac_nominal", "clock_mhz_measured"):
        if roof.get(key) is not None:
            row[key] = roof[key]
    cb = rec.get("cpu_baseline")
    if cb is not None:
        row["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "seconds", "sample")}
        if "parity" in cb:
            row["parity"] = cb["parity"]
    return row


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help=f"one workload alone (default: {DEFAULT_WORKLOAD}, with the other "
                         "four configurations' record beside it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--flush", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the extra cache-cold timing pass reported beside the warm one")
    ap.add_argument("--list-workloads", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    from exact_attention_49_amd import inputs
    if args.list_workloads:
        for name, w in inputs.WORKLOADS.items():
            print(f"{name}: {w.note}")
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (its work "
              "units, one per (batch | sequence, head), shard over GPUs without any exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy()
        return 0

    import torch

    cpu = None if args.no_cpu_baseline else args.cpu_budget
    name = args.workload or DEFAULT_WORKLOAD
    out = run_workload(inputs.WORKLOADS[name], args.steps, args.warmup, args.flush,
                       not args.no_cold, cpu)
    if args.workload is None:
        # the default run also records the other four configurations: same timing method,
        # at least 20 timed steps (200 for the launch-bound tiny one), no cold pass, and a
        # shorter oracle sample each
        rows = []
        for cname in FIVE_CONFIGS:
            if cname == name:
                rows.append(config_summary(out))
                continue
            torch.cuda.empty_cache()
            steps = max(args.steps, 200 if cname == "tiny_fp16_d64" else 20)
            rec = run_workload(inputs.WORKLOADS[cname], steps, max(args.warmup, 3), args.flush,
                               False, None if cpu is None else min(cpu, 5.0))
            rows.append(config_summary(rec))
            print(f"config {cname}: {rows[-1]['tflops']} TFLOP/s "
                  f"({rows[-1]['avg_launch_us']} us per launch)", file=sys.stderr, flush=True)
        out["configs"] = rows
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
