"""The C ABI from plain C: exact_attention_49_amd/examples/c_abi_demo.c (built with gcc by the
package build, no C++, Python or torch involved) calls attn_fwd and attn_fwd_varlen on device
memory it allocated itself and writes its inputs and outputs to files; here they are checked
against the fp64 oracle on the same inputs, to the forward's bars."""

import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from exact_attention_49_amd import build
from tests.gpu_helpers import assert_close

pytestmark = pytest.mark.gpu


def _load(outdir, name):
    meta = json.load(open(os.path.join(outdir, name + ".json")))
    raw = open(os.path.join(outdir, name + ".bin"), "rb").read()
    arrays = {}
    for key, a in meta["arrays"].items():
        if a["dtype"] == "bf16":
            bits = np.frombuffer(raw, np.uint16, a["count"], a["offset"]).astype(np.uint32) << 16
            arrays[key] = bits.view(np.float32).astype(np.float64)
        elif a["dtype"] == "f32":
            arrays[key] = np.frombuffer(raw, np.float32, a["count"], a["offset"]).astype(np.float64)
        else:
            arrays[key] = np.frombuffer(raw, np.int32, a["count"], a["offset"]).copy()
    return arrays, meta["args"]


def test_c_program_calls_the_library(tmp_path):
    if not os.path.exists(build.C_DEMO):
        build.build_c_demo()
    print("[case] c_abi_demo", flush=True)
    r = subprocess.run([build.C_DEMO, str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert "ok" in r.stdout

    a, args = _load(tmp_path, "dense")
    shape = (args["batch"], args["heads"], args["seqlen"], args["head_dim"])
    q, k, v, o = (a[x].reshape(shape) for x in ("q", "k", "v", "o"))
    o_ref, lse_ref = oracle.attention_dense(q, k, v, args["scale"], bool(args["causal"]),
                                            args["window_left"], args["window_right"])
    assert_close(o, a["lse"].reshape(shape[:3]), o_ref, lse_ref, torch.bfloat16, "C dense")

    a, args = _load(tmp_path, "varlen")
    shape = (args["heads"], args["total_tokens"], args["head_dim"])
    q, k, v, o = (a[x].reshape(shape) for x in ("q", "k", "v", "o"))
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, a["cu_seqlens"], args["scale"],
                                             bool(args["causal"]), args["window_left"],
                                             args["window_right"])
    assert_close(o, a["lse"].reshape(shape[:2]), o_ref, lse_ref, torch.bfloat16, "C varlen")
