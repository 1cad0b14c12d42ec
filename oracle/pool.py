"""Process-pool drivers of the fp64 oracle (test infrastructure only).

Only the tests and the benchmark's CPU-baseline leg use this module. It holds
none of the method's arithmetic: every result comes from an unchanged call of
``oracle.attention`` or ``oracle.attention_backward`` on a group of one head's
query rows, with the rows' global positions. Under the causal rule (key j is
allowed for query i iff j <= i) the keys after a group's last row contribute
exp(-inf) = 0, so a group is passed only the key prefix its last row can see:
the result is the same. K and V reach the worker processes through float32
.npy files (exact for bfloat16 and float32 inputs) that each worker
memory-maps and widens to float64 once per KV head.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile
import time

import numpy as np

# Query rows per oracle call inside a task (keys truncated per group).
GROUP_ROWS = 64


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class _Progress:
    """Prints how many oracle tasks are done, at most every 20 seconds."""

    def __init__(self, total: int, what: str):
        self.total, self.what, self.done = total, what, 0
        self.t0 = self.last = time.perf_counter()

    def step(self):
        self.done += 1
        now = time.perf_counter()
        if now - self.last >= 20.0 or self.done == self.total:
            self.last = now
            print(f"    {self.what}: {self.done}/{self.total} tasks, {now - self.t0:.0f} s",
                  flush=True)


# Per-worker cache of float64 K / V planes: {(path, kv_head): array}.
_KV64: dict = {}
_KV64_BYTES = 3 << 30                # bound on the cache of one worker


def _kv64(path: str, g: int) -> np.ndarray:
    key = (path, g)
    if key not in _KV64:
        plane = np.load(path, mmap_mode="r")[g]
        while _KV64 and sum(a.nbytes for a in _KV64.values()) + plane.size * 8 > _KV64_BYTES:
            _KV64.pop(next(iter(_KV64)))
        _KV64[key] = np.asarray(plane, dtype=np.float64)
    return _KV64[key]


def _rows_task(args):
    """Oracle rows [sel] of one head: groups of GROUP_ROWS sorted rows, each
    against the key prefix its last row can see (all keys if not causal)."""
    from . import fp64 as oracle
    h, g, sel, q_rows, q_pos, causal, scale, kpath, vpath = args
    k = _kv64(kpath, g)
    v = _kv64(vpath, g)
    R, D = q_rows.shape
    out = np.zeros((R, D))
    lse = np.zeros(R)
    for i in range(0, R, GROUP_ROWS):
        pos = q_pos[i:i + GROUP_ROWS]
        n_keys = int(pos.max()) + 1 if causal else k.shape[0]
        o, l_ = oracle.attention(q_rows[None, None, i:i + GROUP_ROWS],
                                 k[None, None, :n_keys], v[None, None, :n_keys],
                                 causal=causal, scale=scale, q_pos=pos)
        out[i:i + len(pos)] = o[0, 0]
        lse[i:i + len(pos)] = l_[0, 0]
    return h, sel, out, lse


def pooled_attention(q, k, v, *, causal, rows, scale=None, n_workers=None, kv_head_of_q=None):
    """Oracle rows for every head of batch 0.

    q: [1, Hq, S, D], k/v: [1, Hkv, S, D] (torch CPU tensors or numpy) in
    sequence order; rows: [Hq, R] sequence positions to check per head
    (sorted ascending). Returns (out [Hq, R, D], lse [Hq, R]) in float64.
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
    kv = (list(kv_head_of_q) if kv_head_of_q is not None
          else [h // (Hq // Hkv) for h in range(Hq)])
    rows = np.asarray(rows, np.int64)
    assert np.all(np.diff(rows, axis=1) > 0), "rows must be sorted and distinct per head"
    R = rows.shape[1]
    n = n_workers or workers()
    # Tasks: each head's sorted rows cut into contiguous slices (at least
    # 4 tasks per worker), queued heaviest (latest rows) first.
    slices = max(1, min(R // GROUP_ROWS, -(-4 * n // Hq)))
    tmp = tempfile.mkdtemp(prefix="ra_oracle_")
    try:
        kpath, vpath = os.path.join(tmp, "k.npy"), os.path.join(tmp, "v.npy")
        np.save(kpath, np.ascontiguousarray(k[0], dtype=np.float32))
        np.save(vpath, np.ascontiguousarray(v[0], dtype=np.float32))
        tasks = []
        for g in sorted(set(kv)):            # heads of one KV head in a row: cache reuse
            for h in (hh for hh in range(Hq) if kv[hh] == g):
                for sel in np.array_split(np.arange(R), slices):
                    r = rows[h, sel]
                    tasks.append((h, g, sel, np.ascontiguousarray(q[0, h, r], dtype=np.float32),
                                  r, causal, scale, kpath, vpath))
        if slices > 1:
            tasks.sort(key=lambda t: -int(t[4][-1]))
        out = np.zeros((Hq, R, D))
        lse = np.zeros((Hq, R))
        env = {"OPENBLAS_NUM_THREADS": "1", "OMP_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}
        old = {key: os.environ.get(key) for key in env}
        os.environ.update(env)
        try:
            with cf.ProcessPoolExecutor(max_workers=min(n, len(tasks)),
                                        mp_context=mp.get_context("spawn")) as ex:
                prog = _Progress(len(tasks), "oracle rows")
                for h, sel, o, l_ in ex.map(_rows_task, tasks):
                    out[h, sel], lse[h, sel] = o, l_
                    prog.step()
        finally:
            for key, val in old.items():
                if val is None:
                    os.environ.pop(key, None)
                else:
                    os.environ[key] = val
        return out, lse
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _bwd_task(args):
    """oracle.attention_backward of one head's rows against the key prefix the
    group's last row can see: the rows' dq, and the rows' contributions to
    dk, dv of the keys at positions >= key0 (zero-padded to the key range)."""
    from . import fp64_bwd as oracle
    h, sel, q_rows, dout_rows, q_pos, scale, key0, S, kpath, vpath, g = args
    k = _kv64(kpath, g)
    v = _kv64(vpath, g)
    n_keys = int(q_pos.max()) + 1
    dq, dk, dv = oracle.attention_backward(q_rows[None, None], k[None, None, :n_keys],
                                           v[None, None, :n_keys], dout_rows[None, None],
                                           causal=True, scale=scale, q_pos=q_pos)
    L = S - key0
    dk_s = np.zeros((L, dq.shape[-1]))
    dv_s = np.zeros((L, dq.shape[-1]))
    if n_keys > key0:
        dk_s[:n_keys - key0] = dk[0, 0, key0:n_keys]
        dv_s[:n_keys - key0] = dv[0, 0, key0:n_keys]
    return h, sel, dq[0, 0], dk_s, dv_s


def pooled_backward(q, k, v, dout, *, rows, key0, scale=None, n_workers=None):
    """Causal-attention gradients on a subset, float64, batch 0, sequence order.

    rows: [Hq, R] sorted distinct query rows per head that include every row
    >= key0. Returns dq [Hq, R, D] of those rows (exact: a dq row needs only
    its own scores) and dk, dv [Hkv, S - key0, D] of the keys at positions
    key0..S-1 (exact: under the causal rule only queries at positions >= key0
    see those keys, and all of them are among the rows)."""
    import torch
    as_np = (lambda t: t.float().numpy()) if isinstance(q, torch.Tensor) else np.asarray
    q, k, v, dout = as_np(q), as_np(k), as_np(v), as_np(dout)
    Hq, S, D = q.shape[1:]
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, np.int64)
    for h in range(Hq):
        assert np.all(np.isin(np.arange(key0, S), rows[h])), "every row >= key0 is needed"
    R = rows.shape[1]
    group = Hq // Hkv
    tmp = tempfile.mkdtemp(prefix="ra_oracle_bwd_")
    try:
        kpath, vpath = os.path.join(tmp, "k.npy"), os.path.join(tmp, "v.npy")
        np.save(kpath, np.ascontiguousarray(k[0], dtype=np.float32))
        np.save(vpath, np.ascontiguousarray(v[0], dtype=np.float32))
        tasks = []
        for h in range(Hq):
            for i in range(0, R, GROUP_ROWS):
                sel = np.arange(i, min(R, i + GROUP_ROWS))
                r = rows[h, sel]
                tasks.append((h, sel, np.ascontiguousarray(q[0, h, r], dtype=np.float32),
                              np.ascontiguousarray(dout[0, h, r], dtype=np.float32), r, scale,
                              key0, S, kpath, vpath, h // group))
        dq = np.zeros((Hq, R, D))
        dk = np.zeros((Hkv, S - key0, D))
        dv = np.zeros((Hkv, S - key0, D))
        env = {"OPENBLAS_NUM_THREADS": "1", "OMP_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}
        old = {key: os.environ.get(key) for key in env}
        os.environ.update(env)
        try:
            with cf.ProcessPoolExecutor(max_workers=min(n_workers or workers(), len(tasks)),
                                        mp_context=mp.get_context("spawn")) as ex:
                prog = _Progress(len(tasks), "oracle gradients")
                for h, sel, dq_h, dk_s, dv_s in ex.map(_bwd_task, tasks):
                    dq[h, sel] = dq_h
                    dk[h // group] += dk_s
                    dv[h // group] += dv_s
                    prog.step()
        finally:
            for key, val in old.items():
                if val is None:
                    os.environ.pop(key, None)
                else:
                    os.environ[key] = val
        return dq, dk, dv
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
