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

