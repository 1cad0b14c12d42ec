"""Build the gfx950 shared library ``libringattn.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into one shared object next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libringattn.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "aux_kernels.hip", "probe.hip", "noalloc.hip",
           "api.cpp"]
# Per-source extra flags. The backward kernels read their S and dP MFMA
# results with the VALU; by default the backend gave those results AGPRs and
# copied 32 of them to VGPRs at every loop iteration. The VGPR form of the
# MFMA instructions writes them where the VALU reads them (bit-identical
# results, no spills).
EXTRA = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile all sources (in parallel) and link ``libringattn.so``; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    errors = []
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(line for line in out.splitlines() if "packed-fp32-ops" not in line)
        if p.returncode != 0:
            errors.append(f"{' '.join(cmd)}\n{out}")
        elif verbose and out.strip():
            print(out, flush=True)
    if errors:
        raise RuntimeError("HIP compilation failed:\n" + "\n\n".join(errors))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
