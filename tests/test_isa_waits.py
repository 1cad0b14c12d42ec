"""Static checks on the gfx950 assembly of the attention kernels (CPU only).

The kernels issue their LDS operand reads by inline asm and wait for them
with hand-counted ``s_waitcnt lgkmcnt(N)``. Two mistakes break that silently
and show up on the GPU only as wrong numbers:

* a use of a register that an inline-asm LDS read is still writing: the
  hardware writes it when the read returns, the compiler takes it as
  written at the read statement, so a wait that does not name the register
  lets uses move above it;
* a compiler-issued LGKM operation (an LDS instruction of its own, e.g. a
  cross-lane shuffle, or a scalar memory load) in flight when a counted
  wait executes: it takes one of the counted slots, so the wait can retire
  before the read it was written for.

Both are checked on the code the library is actually built from (same
flags as the build script), one kernel function at a time, scanning the
instruction stream in program order.
"""
import os
import re
import shutil
import subprocess

import pytest

from ring_context_parallelism_flash_amd import build as ra_build

HIPCC = ra_build.HIPCC
pytestmark = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC),
                                reason="hipcc not available")

KERNEL_SOURCES = ("attn_fwd.hip", "attn_bwd.hip")
_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            for r in range(int(m.group(4)), int(m.group(5)) + 1):
                out.add((m.group(3), r))
    return out


def _kernels(asm):
    """{kernel symbol: [instruction lines]} for every kernel of the module."""
    names = re.findall(r"^\s+\.name:\s+(\S+)", asm, flags=re.M)
    out = {}
    for name in names:
        m = re.search(r"^" + re.escape(name) + r":[^\n]*\n(.*?)^\s*s_endpgm", asm, flags=re.S | re.M)
        if m:
            out[name] = m.group(1).split("\n")
    return out


def _scan(lines):
    """Hazards of both kinds, as (line, text) pairs."""
    hazards = []
    in_asm = False
    outstanding = []   # LGKM operations in issue order: (is_asm_read, dst registers)
    for i, raw in enumerate(lines):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        op = s.split()[0]
        m = re.match(r"s_waitcnt\s+(.*)", s)
        if m:
            lg = re.search(r"lgkmcnt\((\d+)\)", m.group(1))
            if lg:
                n = int(lg.group(1))
                if in_asm and n > 0 and any(not a for a, _ in outstanding):
                    hazards.append((i, f"counted wait lgkmcnt({n}) with a compiler LGKM op in flight"))
                outstanding = outstanding[len(outstanding) - n:] if n else []
            continue
        if op.startswith("ds_"):
            dst = _regs(s.split(None, 1)[1].split(",")[0]) if in_asm and op.startswith("ds_read") else set()
            outstanding.append((in_asm and op.startswith("ds_read"), dst))
            continue
        if op.startswith("s_load") or op.startswith("s_buffer_load"):
            outstanding.append((False, set()))
            continue
        if outstanding and " " in s:
            used = _regs(s.split(None, 1)[1])
            for is_read, dst in outstanding:
                if is_read and dst & used:
                    hazards.append((i, f"'{s}' uses a register an asm LDS read is still writing"))
                    break
    return hazards


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")
    out = {}
    for src in KERNEL_SOURCES:
        path = d / (src + ".s")
        cmd = [HIPCC, *ra_build.FLAGS, *ra_build.EXTRA.get(src, []), "--cuda-device-only", "-S",
               "-x", "hip", os.path.join(ra_build.CSRC, src), "-o", str(path)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[src] = path.read_text()
    return out


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_wait_hazards(assembly, src):
    kernels = _kernels(assembly[src])
    assert any("attn_" in k for k in kernels), "no attention kernel found in the assembly"
    found = {k: _scan(body) for k, body in kernels.items()}
    bad = {k: h for k, h in found.items() if h}
    assert not bad, "\n".join(f"{k}: {h[:3]}" for k, h in bad.items())


def test_scanner_flags_both_hazard_kinds():
    """The scanner itself: a use before the counted wait, and a compiler
    shuffle inside a counted window, are both reported; the correct order is not."""
    read = [";;#ASMSTART", "ds_read_b128 v[10:13], v1 offset:16", ";;#ASMEND"]
    wait0 = [";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND"]
    wait1 = [";;#ASMSTART", "s_waitcnt lgkmcnt(1)", ";;#ASMEND"]
    use = ["v_fma_f32 v20, v11, s2, v21"]
    assert _scan(read + wait0 + use) == []
    assert len(_scan(read + use + wait0)) == 1
    shuffle = ["ds_bpermute_b32 v30, v31, v32"]
    assert len(_scan(read + shuffle + wait1)) == 1
    assert _scan(read + wait1) == []
