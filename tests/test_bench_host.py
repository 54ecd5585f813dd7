"""Host-side checks of bench.py's bookkeeping (no GPU)."""

import os

import bench

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "exact_attention_49_amd", "csrc")


def test_every_kernel_source_belongs_to_a_family():
    """A recorded HBM-traffic figure is tied to the hash of its kernel family's sources, so a
    source file missing from every family could change a kernel without invalidating it."""
    listed = {f for files in bench.KERNEL_SOURCES.values() for f in files}
    on_disk = {f for f in os.listdir(CSRC) if f.endswith((".h", ".hip"))}
    assert on_disk == listed


def test_family_hashes_differ_and_are_stable():
    hashes = {fam: bench.kernel_source_hash(fam) for fam in bench.KERNEL_SOURCES}
    assert len(set(hashes.values())) == len(hashes)
    assert hashes == {fam: bench.kernel_source_hash(fam) for fam in bench.KERNEL_SOURCES}


def test_visible_pairs_closed_forms():
    n = 300
    assert bench.visible_pairs(n, False, -1, -1) == n * n
    assert bench.visible_pairs(n, True, -1, -1) == n * (n + 1) // 2
    # causal with a left window of w: row i sees min(i, w) + 1 keys
    w = 17
    assert bench.visible_pairs(n, True, w, 0) == sum(min(i, w) + 1 for i in range(n))


def test_kernel_names_mirror_the_dispatch_thresholds():
    """bench.py names the kernel the library launches: the ping-pong kernel at d = 128 once
    the 256-row grid reaches 256 workgroups (384 under a causal or window mask)."""
    from exact_attention_49_amd import inputs

    def w(**kw):
        base = dict(name="t", heads=8, head_dim=128, dtype="bf16", causal=False, seed=1,
                    batch=1, seqlen=8192)
        base.update(kw)
        return inputs.Workload(**base)

    assert bench.kernel_name(w()) == "attn_fwd_pp_kernel"                    # 256 tiles
    assert bench.kernel_name(w(heads=4)) == "attn_fwd_kernel"                # 128 tiles
    assert bench.kernel_name(w(causal=True)) == "attn_fwd_kernel"            # 256 masked
    assert bench.kernel_name(w(causal=True, heads=12)) == "attn_fwd_pp_kernel"  # 384 masked
    assert bench.kernel_name(w(window_left=1024)) == "attn_fwd_kernel"
    assert bench.kernel_name(w(window_left=8192)) == "attn_fwd_pp_kernel"    # covers every key
    assert bench.kernel_name(w(head_dim=64)) == "attn_fwd_kernel"
    assert bench.kernel_name(w(head_dim=512)) == "attn_fwd_wide_kernel"
    named = {n: bench.kernel_name(x) for n, x in inputs.WORKLOADS.items() if not x.varlen}
    assert named["causal_bf16_d128_n8192"] == "attn_fwd_pp_kernel"
    assert named["causal_bf16_d128_n2048"] == "attn_fwd_pp_kernel"
    assert named["dense_fp16_d512_n4096"] == "attn_fwd_wide_kernel"
    assert named["fp8_causal_d128_n8192"] == "attn_fwd_fp8_kernel"
