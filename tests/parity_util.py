"""Shared helpers for the GPU parity tests: tolerances, comparison, and a
process pool that runs the (unchanged) fp64 oracle one query head per task.

The pool only distributes work: each task calls ``oracle.attention`` on one
head's query rows, with the rows' global positions, against that head's full
K and V. K and V reach the workers through float32 .npy files (exact for
bfloat16 and float32 inputs) that the workers memory-map.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

# Tolerances: bf16 inputs with fp32 accumulation, and fp32 inputs.
TOL_BF16 = dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3)
TOL_F32 = dict(max_abs=1e-4, mean_abs=1e-4, lse=1e-4)


def tol_for(dtype_name: str):
    return TOL_F32 if dtype_name == "f32" else TOL_BF16


def compare(out, lse, ref_out, ref_lse, tol, what=""):
    """Element-wise comparison in float64; returns the error summary."""
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
    assert np.all(lse[~fin] == -np.inf), f"{what}: empty rows must have lse=-inf"
    err = np.abs(out - ref_out)
    lerr = np.abs(lse[fin] - ref_lse[fin]) if fin.any() else np.zeros(1)
    s = dict(max_abs=float(err.max()) if err.size else 0.0,
             mean_abs=float(err.mean()) if err.size else 0.0,
             lse_max=float(lerr.max()))
    print(f"  {what}: out max {s['max_abs']:.3e} mean {s['mean_abs']:.3e} "
          f"lse max {s['lse_max']:.3e}", flush=True)
    assert s["max_abs"] <= tol["max_abs"], (what, s)
    assert s["mean_abs"] <= tol["mean_abs"], (what, s)
    assert s["lse_max"] <= tol["lse"], (what, s)
    return s


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _head_task(args):
    import oracle
    h, g, q_rows, q_pos, causal, scale, kpath, vpath = args
    k = np.load(kpath, mmap_mode="r")[g]
    v = np.load(vpath, mmap_mode="r")[g]
    out, lse = oracle.attention(q_rows[None, None], np.asarray(k)[None, None],
                                np.asarray(v)[None, None], causal=causal, scale=scale,
                                q_pos=q_pos)
    return h, out[0, 0], lse[0, 0]


def pooled_attention(q, k, v, *, causal, rows, scale=None, n_workers=None):
    """Oracle rows for every head of batch 0.

    q: [1, Hq, S, D], k/v: [1, Hkv, S, D] (torch CPU tensors or numpy);
    rows: [Hq, R] sequence positions to check per head (sorted).
    Returns (out [Hq, R, D], lse [Hq, R]) in float64.
    """
    import torch
    if isinstance(q, torch.Tensor):
        q = q.float().numpy()
        k = k.float().numpy()
        v = v.float().numpy()
    assert q.shape[0] == 1
    Hq, S, D = q.shape[1:]
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, np.int64)
    tmp = tempfile.mkdtemp(prefix="ra_oracle_")
    try:
        kpath, vpath = os.path.join(tmp, "k.npy"), os.path.join(tmp, "v.npy")
        np.save(kpath, np.ascontiguousarray(k[0], dtype=np.float32))
        np.save(vpath, np.ascontiguousarray(v[0], dtype=np.float32))
        tasks = [(h, h // (Hq // Hkv), np.ascontiguousarray(q[0, h, rows[h]], dtype=np.float32),
                  rows[h], causal, scale, kpath, vpath) for h in range(Hq)]
        out = np.zeros((Hq, rows.shape[1], D))
        lse = np.zeros((Hq, rows.shape[1]))
        n = n_workers or workers()
        old = os.environ.get("OPENBLAS_NUM_THREADS")
        os.environ["OPENBLAS_NUM_THREADS"] = "1"
        try:
            with cf.ProcessPoolExecutor(max_workers=min(n, Hq),
                                        mp_context=mp.get_context("spawn")) as ex:
                for h, o, l_ in ex.map(_head_task, tasks):
                    out[h], lse[h] = o, l_
        finally:
            if old is None:
                os.environ.pop("OPENBLAS_NUM_THREADS", None)
            else:
                os.environ["OPENBLAS_NUM_THREADS"] = old
        return out, lse
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def boundary_rows(S: int, n_chunks: int) -> np.ndarray:
    """First and last row of every one of ``n_chunks`` equal chunks."""
    c = S // n_chunks
    return np.unique(np.concatenate([np.arange(n_chunks) * c, np.arange(1, n_chunks + 1) * c - 1]))


def check_rows(S: int, Hq: int, n_random: int, seed: int, n_chunks: int) -> np.ndarray:
    """[Hq, R] rows per head: seeded random rows plus every chunk's boundary rows."""
    from workloads import sample_rows
    b = boundary_rows(S, n_chunks)
    out = []
    for h in range(Hq):
        r = np.union1d(sample_rows(S, n_random, seed, h), b)
        out.append(r)
    R = min(len(r) for r in out)
    return np.stack([r[:R] for r in out])
