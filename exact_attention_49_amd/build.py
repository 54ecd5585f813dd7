"""Build the gfx950 HIP library in-tree: exact_attention_49_amd/libexact_attn.so.

    python -m exact_attention_49_amd.build

Each csrc/*.hip file is compiled by hipcc for gfx950 in parallel, then linked into one shared
library.  Packed-fp32 VALU instructions are disabled for the device code.  The plain-C example
consumer (examples/c_abi_demo.c) is then compiled against the library with gcc.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libexact_attn.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

# The wide-head-dim kernels keep the output accumulators in AGPRs through inline assembly and
# want every compiler-selected MFMA in VGPR form.
EXTRA_FLAGS = {
    "attn_fwd_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    "attn_fwd_d512.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}


def _compile(src: str, obj: str) -> str:
    cmd = [HIPCC, *CFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in (r.stderr or "").splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return err


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libexact_attn.so (always rebuilds)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = {ex.submit(_compile, os.path.join(CSRC, s), o): s for s, o in zip(srcs, objs)}
        for f in cf.as_completed(futs):
            msg = f.result()
            if verbose and msg:
                print(f"[{futs[f]}]\n{msg}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_c_demo()
    return LIB


C_DEMO_SRC = os.path.join(PKG, "examples", "c_abi_demo.c")
C_DEMO = os.path.join(PKG, "c_abi_demo")


def build_c_demo() -> str:
    """Compile the plain-C example consumer of the library (gcc, C11) next to the library."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", "/opt/rocm/include", C_DEMO_SRC, "-L", PKG, "-lexact_attn",
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,/opt/rocm/lib",
           "-o", C_DEMO]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {C_DEMO_SRC}:\n{r.stderr}")
    return C_DEMO


if __name__ == "__main__":
    print(build(verbose=True))
