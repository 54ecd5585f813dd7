"""CPU-side checks of the C-ABI library: it loads, it exports every function the header
declares, the binding's signatures cover them, and argument validation rejects bad calls on
the host before any HIP call (no kernel is ever launched here)."""

import ctypes
import os
import re
import subprocess

import pytest

from exact_attention_49_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exact_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from exact_attention_49_amd import build
        build.build()
    return binding.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    fns = header_functions()
    assert {"attn_fwd", "attn_fwd_varlen", "attn_status_string"} <= set(fns)


def test_library_exports_every_header_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for fn in header_functions():
        assert fn in exported, fn
        assert fn in binding.EXPORTED_SYMBOLS, fn
        assert isinstance(getattr(lib, fn), ctypes._CFuncPtr)


_CTYPE_OF = {"int": ctypes.c_int, "float": ctypes.c_float, "size_t": ctypes.c_size_t}


def header_signatures():
    """{name: (return type, [argument types])} parsed from the header, as ctypes types."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    sigs = {}
    for ret, name, params in re.findall(r"^([A-Za-z_][\w \*]*?)\s*\b(attn_\w+)\s*\(([^)]*)\)\s*;",
                                        text, flags=re.M):
        def ctype(decl):
            decl = decl.strip()
            if decl == "void" or not decl:
                return None
            if "*" in decl:
                return ctypes.c_char_p if decl.startswith("const char") else ctypes.c_void_p
            return _CTYPE_OF[decl.rsplit(None, 1)[0].replace("const ", "")]
        args = [ctype(p) for p in params.split(",")]
        sigs[name] = (ctype(ret + " x" if "*" not in ret else ret), [a for a in args if a])
    return sigs


def test_binding_signatures_match_the_header():
    sigs = header_signatures()
    assert set(sigs) == set(header_functions())
    for name, (ret, args) in sigs.items():
        b_ret, b_args = binding.EXPORTED_SYMBOLS[name]
        assert b_ret == ret, name
        assert b_args == args, name


def test_status_strings(lib):
    for code, name in binding.STATUS.items():
        assert lib.attn_status_string(code).decode().startswith(name)
    assert lib.attn_status_string(12345) == b"unknown status"
    assert lib.attn_last_hip_error() == 0


A = 1 << 20          # a fake, 16-byte aligned address: validation never dereferences it
SCALE = 0.125


def call_dense(lib, q=A, k=A, v=A, o=A, lse=None, b=1, h=1, n=16, d=64, dtype=1,
               scale=SCALE, causal=0, wl=-1, wr=-1):
    return lib.attn_fwd(q, k, v, o, lse, b, h, n, d, dtype, scale, causal, wl, wr, None)


def call_varlen(lib, q=A, k=A, v=A, o=A, lse=None, cu=A, ns=2, maxs=8, total=16, h=1, d=64,
                dtype=1, scale=SCALE, causal=0, wl=-1, wr=-1):
    return lib.attn_fwd_varlen(q, k, v, o, lse, cu, ns, maxs, total, h, d, dtype, scale,
                               causal, wl, wr, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(b=-1), 1), (dict(h=-2), 1), (dict(n=-1), 1),
    (dict(d=96), 2), (dict(d=32), 2), (dict(d=1024), 2),
    (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(q=A + 8), 4), (dict(o=A + 2), 4), (dict(lse=A + 2), 4),
    (dict(scale=0.0), 1), (dict(scale=-1.0), 1), (dict(scale=float("inf")), 1),
    (dict(scale=float("nan")), 1),
    (dict(causal=2), 1), (dict(wl=-2), 1), (dict(wr=-5), 1),
    # one (sequence, head) of K or V must stay below 2 GiB (32-bit byte offsets)
    (dict(n=1 << 21, d=512), 5), (dict(n=1 << 23, d=128), 5),
])
def test_dense_rejects_bad_arguments(lib, kw, status):
    assert call_dense(lib, **kw) == status


@pytest.mark.parametrize("kw", [dict(b=0), dict(h=0), dict(n=0)])
def test_dense_empty_problem_is_a_no_op(lib, kw):
    # nothing to compute: returns OK without launching (pointers are never touched)
    assert call_dense(lib, q=None, k=None, v=None, o=None, **kw) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), 1), (dict(cu=A + 2), 4), (dict(ns=-1), 1), (dict(total=-1), 1),
    (dict(maxs=0), 1), (dict(maxs=17), 1), (dict(h=-1), 1), (dict(d=80), 2), (dict(dtype=7), 3),
    (dict(q=None), 1), (dict(v=A + 4), 4), (dict(scale=0.0), 1), (dict(wl=-3), 1),
    (dict(maxs=1 << 21, total=1 << 21, d=512), 5),
])
def test_varlen_rejects_bad_arguments(lib, kw, status):
    assert call_varlen(lib, **kw) == status


@pytest.mark.parametrize("kw", [dict(ns=0), dict(total=0), dict(h=0)])
def test_varlen_empty_problem_is_a_no_op(lib, kw):
    assert call_varlen(lib, q=None, k=None, v=None, o=None, cu=None, **kw) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(binding.AttnError, match="GPU tensor"):
        binding.attn_fwd(x, x, x)


# ---- split-KV entry points (host-side validation and workspace sizing only) ----------------

def call_dense_split(lib, ns=2, ws=A, wsb=1 << 30, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=None, b=1, h=1, hkv=None, n=4096, d=128, dtype=1,
                scale=SCALE, causal=0, wl=-1, wr=-1)
    args.update(kw)
    hkv = args["h"] if args["hkv"] is None else args["hkv"]
    return lib.attn_fwd_splitkv(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                args["b"], args["h"], hkv, args["n"], args["d"], args["dtype"],
                                args["scale"], args["causal"], args["wl"], args["wr"], ns, ws,
                                wsb, None)


def test_splitkv_workspace_size_formula(lib):
    # ns partial rows of d fp32 values plus ns LSE values per row, each part 256-byte aligned
    def expect(rows, d, ns):
        up = lambda x: (x + 255) // 256 * 256  # noqa: E731
        return up(ns * rows * d * 4) + up(ns * rows * 4)
    for causal, wl in ((0, -1), (1, -1), (1, 100)):  # the mask only matters for ns = 0
        assert lib.attn_fwd_splitkv_workspace_size(2, 3, 1000, 128, 4, causal, wl) == \
            expect(6000, 128, 4)
        assert lib.attn_fwd_splitkv_workspace_size(1, 1, 77, 64, 3, causal, wl) == \
            expect(77, 64, 3)
    assert lib.attn_fwd_varlen_splitkv_workspace_size(5, 300, 1000, 4, 256, 2) == \
        expect(4000, 256, 2)
    assert lib.attn_fwd_splitkv_workspace_size(1, 1, 4096, 128, 1, 0, -1) == 0    # one split
    assert lib.attn_fwd_splitkv_workspace_size(1, 1, 4096, 96, 2, 0, -1) == 0     # bad head dim
    assert lib.attn_fwd_splitkv_workspace_size(1, 1, 4096, 128, 65, 0, -1) == 0   # too many
    assert lib.attn_fwd_splitkv_workspace_size(0, 1, 4096, 128, 2, 0, -1) == 0    # empty


def test_splitkv_automatic_count(lib):
    for causal in (0, 1):
        # a grid that fills the chip needs no split; a single long head does
        assert lib.attn_fwd_splitkv_num_splits(2, 32, 8192, 128, causal, -1) == 1
        s = lib.attn_fwd_splitkv_num_splits(1, 1, 16384, 128, causal, -1)
        assert 2 <= s <= 64
        assert lib.attn_fwd_splitkv_workspace_size(1, 1, 16384, 128, 0, causal, -1) == \
            lib.attn_fwd_splitkv_workspace_size(1, 1, 16384, 128, s, causal, -1)
        # never fewer than eight key tiles per split
        assert lib.attn_fwd_splitkv_num_splits(1, 1, 256, 128, causal, -1) == 1
        assert lib.attn_fwd_splitkv_num_splits(1, 1, 4096, 128, causal, -1) == 8
    assert lib.attn_fwd_varlen_splitkv_num_splits(2, 8192, 9000, 1, 64) >= 2
    # enough work items for every CU's resident share: four small-shape workgroups per CU at
    # d = 64 (2 heads x 128 q-tiles -> 4 splits), two at d = 128 (-> 2 splits)
    assert lib.attn_fwd_splitkv_num_splits(1, 2, 16384, 64, 0, -1) == 4
    assert lib.attn_fwd_splitkv_num_splits(1, 2, 16384, 128, 0, -1) == 2
    # causal without a left window over at most 3 (batch, head) pairs: twice the items
    assert lib.attn_fwd_splitkv_num_splits(1, 2, 16384, 64, 1, -1) == 8
    assert lib.attn_fwd_splitkv_num_splits(1, 2, 16384, 128, 1, -1) == 4
    assert lib.attn_fwd_splitkv_num_splits(1, 2, 16384, 128, 1, 16384) == 4   # no window
    assert lib.attn_fwd_splitkv_num_splits(1, 3, 16384, 128, 1, -1) == 3
    # ... while a split of the longest range keeps 16 key tiles (128 tiles: 8, not 16)
    assert lib.attn_fwd_splitkv_num_splits(1, 1, 8192, 128, 1, -1) == 8
    assert lib.attn_fwd_splitkv_num_splits(1, 1, 8192, 128, 0, -1) == 8
    # ... but not with a sliding window, more pairs, or packed sequences
    assert lib.attn_fwd_splitkv_num_splits(1, 2, 16384, 128, 1, 1024) == 2
    assert lib.attn_fwd_splitkv_num_splits(2, 2, 8192, 128, 1, -1) == 2
    assert lib.attn_fwd_splitkv_num_splits(1, 8, 4096, 128, 1, -1) == 2
    assert lib.attn_fwd_splitkv_num_splits(1, 8, 4096, 128, 0, -1) == 2
    assert lib.attn_fwd_varlen_splitkv_num_splits(1, 16384, 16384, 2, 128) == 2


@pytest.mark.parametrize("kw,status", [
    (dict(ns=-1), 1), (dict(ns=65), 1),                      # split count
    (dict(ws=None), 1), (dict(ws=A + 64), 1), (dict(wsb=1024), 1),   # workspace
    (dict(q=None), 1), (dict(d=96), 2), (dict(dtype=5), 3), (dict(o=A + 2), 4),
    (dict(h=8, hkv=3), 1), (dict(h=8, hkv=0), 1), (dict(h=4, hkv=8), 1),   # head grouping
])
def test_splitkv_rejects_bad_arguments(lib, kw, status):
    assert call_dense_split(lib, **kw) == status


def test_splitkv_one_split_needs_no_workspace(lib):
    # with one split the plain kernels run; validation still happens on the host first
    assert call_dense_split(lib, ns=1, ws=None, wsb=0, d=96) == 2
    assert call_dense_split(lib, ns=0, ws=None, wsb=0, b=0) == 0   # empty problem


# ---- grouped-query entry points (host-side validation only) ----------------------------------

def call_gqa(lib, hq=8, hkv=2, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=None, b=1, n=16, d=64, dtype=1, scale=SCALE, causal=0,
                wl=-1, wr=-1)
    args.update(kw)
    return lib.attn_fwd_gqa(args["q"], args["k"], args["v"], args["o"], args["lse"], args["b"],
                            hq, hkv, args["n"], args["d"], args["dtype"], args["scale"],
                            args["causal"], args["wl"], args["wr"], None)


def call_varlen_gqa(lib, hq=8, hkv=2, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=None, cu=A, ns=2, maxs=8, total=16, d=64, dtype=1,
                scale=SCALE, causal=0, wl=-1, wr=-1)
    args.update(kw)
    return lib.attn_fwd_varlen_gqa(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                   args["cu"], args["ns"], args["maxs"], args["total"], hq, hkv,
                                   args["d"], args["dtype"], args["scale"], args["causal"],
                                   args["wl"], args["wr"], None)


@pytest.mark.parametrize("call", [call_gqa, call_varlen_gqa])
@pytest.mark.parametrize("hq,hkv", [(8, 3), (8, 0), (8, -2), (4, 8), (6, 4)])
def test_gqa_rejects_head_counts_that_do_not_divide(lib, call, hq, hkv):
    assert call(lib, hq=hq, hkv=hkv) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(d=96), 2), (dict(dtype=4), 3), (dict(k=A + 2), 4),
    (dict(causal=3), 1),
])
def test_gqa_other_checks_match_the_plain_calls(lib, kw, status):
    assert call_gqa(lib, **kw) == status
    assert call_varlen_gqa(lib, **kw) == status


def test_gqa_empty_problem_is_a_no_op(lib):
    assert call_gqa(lib, hq=0, hkv=1, q=None, k=None, v=None, o=None) == 0
    assert call_gqa(lib, b=0, q=None, k=None, v=None, o=None) == 0
    assert call_varlen_gqa(lib, ns=0, q=None, k=None, v=None, o=None, cu=None) == 0


def test_binding_gqa_checks_shapes():
    import torch
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(binding.AttnError, match="GPU tensor"):
        binding.attn_fwd_gqa(q, q[:, :2], q[:, :2])


# ---- backward entry points (host-side validation and workspace sizing only) ------------------

def call_bwd(lib, ws=A, wsb=1 << 30, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, b=1, hq=2, hkv=1, n=256,
                d=128, dtype=1, scale=SCALE, causal=1, wl=-1, wr=-1)
    args.update(kw)
    return lib.attn_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"],
                        args["dq"], args["dk"], args["dv"], args["b"], args["hq"], args["hkv"],
                        args["n"], args["d"], args["dtype"], args["scale"], args["causal"],
                        args["wl"], args["wr"], ws, wsb, None)


def call_bwd_varlen(lib, ws=A, wsb=1 << 30, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, cu=A, ns=2, maxs=8,
                total=16, hq=2, hkv=2, d=64, dtype=0, scale=SCALE, causal=0, wl=-1, wr=-1)
    args.update(kw)
    return lib.attn_bwd_varlen(args["q"], args["k"], args["v"], args["o"], args["lse"],
                               args["do"], args["dq"], args["dk"], args["dv"], args["cu"],
                               args["ns"], args["maxs"], args["total"], args["hq"], args["hkv"],
                               args["d"], args["dtype"], args["scale"], args["causal"],
                               args["wl"], args["wr"], ws, wsb, None)


@pytest.mark.parametrize("call", [call_bwd, call_bwd_varlen])
@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1), (dict(q=None), 1), (dict(o=None), 1),
    (dict(d=256), 2), (dict(d=512), 2), (dict(d=96), 2), (dict(dtype=3), 3),
    (dict(do=A + 4), 4), (dict(dq=A + 2), 4), (dict(dv=A + 8), 4), (dict(lse=A + 2), 4),
    (dict(hq=4, hkv=3), 1), (dict(scale=0.0), 1), (dict(causal=2), 1),
    (dict(ws=None), 1), (dict(ws=A + 16), 1), (dict(wsb=4), 1),
])
def test_bwd_rejects_bad_arguments(lib, call, kw, status):
    assert call(lib, **kw) == status


def test_bwd_workspace_size(lib):
    # two fp32 arrays of one value per query row (dPsum, LSE in log2 units), each padded to
    # whole 256-byte granules
    assert lib.attn_bwd_workspace_size(2, 32, 8192) == 2 * (2 * 32 * 8192 * 4)
    assert lib.attn_bwd_workspace_size(1, 3, 5) == 2 * 256      # 60 bytes each
    assert lib.attn_bwd_workspace_size(0, 3, 5) == 0
    assert lib.attn_bwd_varlen_workspace_size(1000, 6) == 2 * 24064
    assert lib.attn_bwd_varlen_workspace_size(0, 6) == 0


def test_bwd_rejects_a_workspace_one_byte_short(lib):
    # b = 1, heads_q = 2, n = 256: 512 query rows, two arrays of 2048 bytes
    need = lib.attn_bwd_workspace_size(1, 2, 256)
    assert need == 4096
    assert call_bwd(lib, wsb=need - 1) == 1
    need_v = lib.attn_bwd_varlen_workspace_size(16, 2)   # 32 rows: two 256-byte arrays
    assert need_v == 512
    assert call_bwd_varlen(lib, wsb=need_v - 1) == 1


def test_binding_bwd_workspace_helpers_match_the_library(lib):
    for args in [(2, 32, 8192), (1, 3, 5), (0, 3, 5), (3, 7, 1000)]:
        assert binding.bwd_workspace_size(*args) == lib.attn_bwd_workspace_size(*args)
    for args in [(1000, 6), (0, 6), (12345, 5)]:
        assert (binding.varlen_bwd_workspace_size(*args)
                == lib.attn_bwd_varlen_workspace_size(*args))


def test_bwd_empty_problem_is_a_no_op(lib):
    assert call_bwd(lib, b=0, ws=None, wsb=0) == 0
    assert call_bwd_varlen(lib, ns=0, ws=None, wsb=0) == 0
    assert call_bwd(lib, b=0, d=256) == 2   # non-size arguments are still checked


# ---- FP8 forward (host-side validation only) -------------------------------------------------

def call_fp8(lib, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=None, dq=None, dk=None, dv=None, b=1, hq=2, hkv=1,
                n=256, d=128, out=1, scale=SCALE, causal=1, wl=-1, wr=-1)
    args.update(kw)
    return lib.attn_fwd_fp8(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dq"],
                            args["dk"], args["dv"], args["b"], args["hq"], args["hkv"], args["n"],
                            args["d"], args["out"], args["scale"], args["causal"], args["wl"],
                            args["wr"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(d=96), 2), (dict(d=512), 2), (dict(out=2), 3),
    (dict(q=A + 8), 4), (dict(o=A + 2), 4), (dict(dq=A + 2), 4), (dict(dv=A + 1), 4),
    (dict(hq=4, hkv=3), 1), (dict(scale=0.0), 1), (dict(wl=-3), 1),
])
def test_fp8_rejects_bad_arguments(lib, kw, status):
    assert call_fp8(lib, **kw) == status


def test_fp8_empty_problem_is_a_no_op(lib):
    assert call_fp8(lib, b=0, q=None, k=None, v=None, o=None) == 0


def test_device_info_rejects_null_pointers(lib):
    assert lib.attn_device_info(0, None, None) == 1


def call_persistent(lib, q=A, k=A, v=A, o=A, lse=None, b=1, h=2, hkv=1, n=16, d=128, dtype=1,
                    scale=SCALE, causal=0, wl=-1, wr=-1):
    return lib.attn_fwd_persistent(q, k, v, o, lse, b, h, hkv, n, d, dtype, scale, causal, wl,
                                   wr, None)


def call_varlen_persistent(lib, cu=A, ns=2, maxs=8, total=16, h=2, hkv=1, d=128, **kw):
    q, k, v, o = (kw.pop(x, A) for x in "qkvo")
    return lib.attn_fwd_varlen_persistent(q, k, v, o, None, cu, ns, maxs, total, h, hkv, d, 1,
                                          SCALE, 0, -1, -1, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), 2), (dict(d=256), 2), (dict(d=96), 2), (dict(hkv=3), 1), (dict(hkv=0), 1),
    (dict(q=None), 1), (dict(dtype=5), 3), (dict(k=A + 8), 4), (dict(scale=0.0), 1),
    (dict(causal=3), 1), (dict(n=1 << 23), 5),
])
def test_persistent_rejects_bad_arguments(lib, kw, status):
    assert call_persistent(lib, **kw) == status


def test_persistent_empty_problem_is_a_no_op(lib):
    assert call_persistent(lib, q=None, k=None, v=None, o=None, n=0) == 0
    assert call_varlen_persistent(lib, q=None, k=None, v=None, o=None, cu=None, ns=0) == 0


@pytest.mark.parametrize("kw,status", [(dict(d=64), 2), (dict(cu=None), 1), (dict(maxs=17), 1),
                                       (dict(hkv=3), 1)])
def test_varlen_persistent_rejects_bad_arguments(lib, kw, status):
    assert call_varlen_persistent(lib, **kw) == status
