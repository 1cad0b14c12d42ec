"""The generated key / query loops (CPU only): each generator, run afresh,
passes its own hazard checks and writes exactly the header the library is
built from, so the committed headers are the generators' output and not
edited by hand."""
import os
import shutil
import subprocess
import sys

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "ring_context_parallelism_flash_amd", "csrc")

GENERATORS = [
    ("gen_fwd_w64.py", "attn_fwd_w64_phases.h"),
    ("gen_bwd_dkdv_w32.py", "attn_bwd_dkdv_loop.h"),
    ("gen_bwd_dq_w64.py", "attn_bwd_dq_w64_loop.h"),
]


@pytest.mark.parametrize("gen,header", GENERATORS)
def test_generator_reproduces_committed_header(tmp_path, gen, header):
    shutil.copy(os.path.join(CSRC, gen), tmp_path / gen)
    r = subprocess.run([sys.executable, str(tmp_path / gen)], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(tmp_path / header) as f:
        fresh = f.read()
    with open(os.path.join(CSRC, header)) as f:
        committed = f.read()
    assert fresh == committed, f"{header} differs from what {gen} writes"
