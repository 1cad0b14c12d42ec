"""Host-side checks of the benchmark's bookkeeping (no GPU)."""
import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_kernel_hash_does_not_depend_on_the_checkout_path(monkeypatch, tmp_path):
    """The counter summaries are keyed by a hash of the kernel sources and
    compile flags; the flags hold include paths, which must enter the hash
    relative to the repository, so a checkout elsewhere hashes the same."""
    from ring_context_parallelism_flash_amd import build as ra_build
    h = bench.kernel_sources_sha256()
    hb = bench.kernel_sources_sha256(bench.BWD_KERNEL_SOURCES)
    other = tmp_path / "elsewhere" / "repo"
    shutil.copytree(os.path.join(ROOT, "ring_context_parallelism_flash_amd", "csrc"),
                    other / "ring_context_parallelism_flash_amd" / "csrc")
    monkeypatch.setattr(ra_build, "FLAGS", [f.replace(ROOT, str(other)) for f in ra_build.FLAGS])
    monkeypatch.setattr(bench, "ROOT", str(other))
    assert any(str(other) in f for f in ra_build.FLAGS)
    assert bench.kernel_sources_sha256() == h
    assert bench.kernel_sources_sha256(bench.BWD_KERNEL_SOURCES) == hb


def test_copy_overlap_counts_time_under_attention(tmp_path):
    """Copy intervals are credited only for the part an attention kernel
    covers; overlapping attention intervals are not double counted."""
    rows = [
        ("attn_fwd_bf16<128>", 100, 200),
        ("attn_fwd_bf16<128>", 150, 260),     # overlaps the first
        ("__amd_rocclr_copyBufferRectAligned", 90, 110),    # 10 of 20 covered
        ("__amd_rocclr_copyBufferRectAligned", 250, 300),   # 10 of 50 covered
        ("__amd_rocclr_copyBufferRectAligned", 400, 430),   # 0 of 30 covered
        ("zigzag_permute_kernel", 0, 1000),                  # neither
    ]
    p = tmp_path / "run_kernel_trace.csv"
    with open(p, "w") as f:
        f.write('"Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for name, a, b in rows:
            f.write(f'"{name}",{a},{b}\n')
    r = bench.copy_overlap(str(p))
    assert r["copies"] == 3 and r["attention_launches"] == 2
    assert abs(r["copy_ms"] - 100e-6) < 1e-12
    assert abs(r["copy_ms_under_attention"] - 20e-6) < 1e-12
    assert abs(r["overlap_frac"] - 0.2) < 1e-12


def test_baseline_rows_cover_chunk_boundaries():
    import numpy as np
    import workloads
    w = workloads.HEADLINE
    rows = bench.baseline_rows(w, 100)
    c = w.S // (2 * w.N)
    assert rows.shape == (w.Hq, 2 * 2 * w.N + 100)
    for r in rows:
        assert np.all(np.diff(r) > 0)
        assert np.all(np.isin(np.arange(2 * w.N) * c, r))
        assert np.all(np.isin(np.arange(1, 2 * w.N + 1) * c - 1, r))
