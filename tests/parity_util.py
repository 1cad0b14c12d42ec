"""Shared helpers for the GPU parity tests: tolerances, comparison and the
rows a large configuration is checked on. The process-pool drivers of the
oracle live in ``oracle.pool`` (re-exported here)."""
from __future__ import annotations

import numpy as np

from oracle.pool import GROUP_ROWS, pooled_attention, pooled_backward, workers  # noqa: F401

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


def boundary_rows(S: int, n_chunks: int) -> np.ndarray:
    """First and last row of every one of ``n_chunks`` equal chunks."""
    c = S // n_chunks
    return np.unique(np.concatenate([np.arange(n_chunks) * c, np.arange(1, n_chunks + 1) * c - 1]))


def check_rows(S: int, Hq: int, n_random: int, seed: int, n_chunks: int,
               fixed=None) -> np.ndarray:
    """[Hq, R] sorted rows per head: every chunk's first and last row (plus
    ``fixed``) for every head, and ``n_random`` seeded rows drawn per head
    from the remaining rows with ``numpy.random.default_rng([seed, h])``.
    Every head gets the same R = len(fixed rows) + n_random, without cutting."""
    b = boundary_rows(S, n_chunks)
    if fixed is not None:
        b = np.union1d(b, np.asarray(fixed, np.int64))
    rest = np.setdiff1d(np.arange(S, dtype=np.int64), b)
    n_random = min(n_random, len(rest))
    out = []
    for h in range(Hq):
        rnd = np.random.default_rng([seed, h]).choice(rest, n_random, replace=False)
        out.append(np.sort(np.concatenate([b, rnd])))
    return np.stack(out)
