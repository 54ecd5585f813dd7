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
