"""Plain fp64 CPU oracle for the ring-attention forward step.

TEST INFRASTRUCTURE ONLY. This module is imported by the tests, by the smoke
check and by the benchmark's CPU-baseline leg, and by nothing else. It shares
no code with the HIP library and does not import it; the GPU path never calls
it. It is written for a reader checking it against the pages by eye, not for
speed.

Sources (cited by page title and section):
  [CP]  "Context Parallelism" (aiwiki): section "Ring attention" (exactness:
        the ring computes full attention with the accumulation distributed),
        section "The causal imbalance" (zigzag: 2N chunks, rank i holds chunks
        i and 2N-1-i), and the ring_attention code listing (per-rank loop,
        running state out=0 / m=-inf / sum=0, source=(rank-step) mod world).
  [SP]  "Sequence Parallelism in Large Language Models: How Megatron-SP,
        DeepSpeed Ulysses, and RingAttention Distribute Long Contexts"
        (llms.blog): section "RingAttention and Blockwise Context
        Parallelism" -- the 4-GPU ring-topology figure, "Algorithmic
        Mechanics" (partitioning into P blocks of s/P, source (i-k) mod P,
        the online-softmax equations for m_new, l_new, O_new) and "Causal
        Masking and Load Balancing" (position i attends to j <= i; striped
        partitioning gives token t to rank t mod P).
  [SCP] "Sequence and Context Parallelism" (praveentn.live): section "What it
        does not change" (the result is identical to single-device attention).

Readings taken where the pages are silent or garbled:
  * softmax scale is 1/sqrt(D), applied to the scores before masking;
  * the causal test is inclusive (j <= i) on GLOBAL sequence positions;
  * lse is the natural-log log-sum-exp of the scaled, allowed scores;
  * a row with no allowed key has lse = -inf and out = 0;
  * the printed O_new multiplies O_block by exp(m_block - m_new)/l_new, which
    is exact only when O_block is the UNNORMALISED block sum
    sum_j exp(s_j - m_block) v_j; that is the reading used in
    ``ring_attention`` and ``merge``;
  * GQA: query head h reads KV head h // (Hq / Hkv) unless a map is given;
  * zigzag keeps a rank's early chunk first in its memory;
  * striped: rank r holds positions r, r+N, r+2N, ... in increasing order.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def to_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU or GPU) torch tensor."""
    if hasattr(x, "detach"):
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _kv_map(Hq: int, Hkv: int, kv_head_of_q=None) -> list[int]:
    if kv_head_of_q is not None:
        return [int(g) for g in kv_head_of_q]
    group = Hq // Hkv
    return [h // group for h in range(Hq)]


def _rows_for_head(rows, h: int, Sq: int) -> np.ndarray:
    if rows is None:
        return np.arange(Sq)
    rows = np.asarray(rows, dtype=np.int64)
    return rows if rows.ndim == 1 else rows[h]


# ---------------------------------------------------------------------------
# The definition: exact softmax attention [SCP "What it does not change";
# CP "Ring attention": "full attention"; SP "Causal Masking": j <= i].
# ---------------------------------------------------------------------------
def attention(q, k, v, *, causal: bool, scale: float | None = None,
              kv_head_of_q=None, q_pos=None, k_pos=None, rows=None):
    """Exact softmax attention in float64.

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D]. ``q_pos`` / ``k_pos`` are the
    global sequence positions of q's and k's rows (default 0..S-1); the
    causal rule allows key j for query i iff k_pos[j] <= q_pos[i]. ``rows``
    selects which query rows to compute: None (all), a 1-D index array used for
    every head, or a 2-D array [Hq, R] of per-head indices.

    Returns (out [B, Hq, R, D], lse [B, Hq, R]) in float64. For each row i:
        s_ij   = scale * <q_i, k_j>            for every allowed j
        lse_i  = log(sum_j exp(s_ij))          (natural log)
        out_i  = sum_j exp(s_ij - lse_i) * v_j
    A row with no allowed key has lse = -inf and out = 0.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kv_map = _kv_map(Hq, Hkv, kv_head_of_q)
    q_pos = np.arange(Sq) if q_pos is None else np.asarray(q_pos, np.int64)
    k_pos = np.arange(Sk) if k_pos is None else np.asarray(k_pos, np.int64)
    R = len(_rows_for_head(rows, 0, Sq))
    out = np.zeros((B, Hq, R, D))
    lse = np.full((B, Hq, R), NEG_INF)
    # Rows are independent; they are taken a few at a time only to bound the
    # size of the [rows, Sk] score matrix (at most 2^24 entries, 128 MiB).
    row_block = max(1, min(256, (1 << 24) // max(Sk, 1)))
    for b in range(B):
        for h in range(Hq):
            g = kv_map[h]
            idx_all = _rows_for_head(rows, h, Sq)
            for r0 in range(0, R, row_block):
                idx = idx_all[r0:r0 + row_block]
                s = scale * (q[b, h, idx] @ k[b, g].T)
                if causal:
                    allowed = k_pos[None, :] <= q_pos[idx][:, None]
                    s = np.where(allowed, s, NEG_INF)
                m = s.max(axis=1)
                ok = m > NEG_INF
                lse_blk = np.full(len(idx), NEG_INF)
                lse_blk[ok] = m[ok] + np.log(
                    np.exp(s[ok] - m[ok, None]).sum(axis=1))
                p = np.zeros_like(s)
                p[ok] = np.exp(s[ok] - lse_blk[ok, None])
                out[b, h, r0:r0 + len(idx)] = p @ v[b, g]
                lse[b, h, r0:r0 + len(idx)] = lse_blk
    return out, lse


# ---------------------------------------------------------------------------
# Sequence layouts [SP "Algorithmic Mechanics" item 1; CP "The causal
# imbalance"].
# ---------------------------------------------------------------------------
def contiguous_order(S: int, N: int) -> np.ndarray:
    """Sequence positions in rank-major memory order for the contiguous split:
    rank i holds block i of P equal blocks of s/P tokens."""
    if S % N:
        raise ValueError("S must be divisible by N")
    return np.arange(S, dtype=np.int64)


def zigzag_order(S: int, N: int) -> np.ndarray:
    """Sequence positions in rank-major memory order for the zigzag split.

    The sequence is cut into 2N chunks of c = S/(2N) tokens and rank i holds
    chunks i and 2N-1-i, the early chunk first. Entry p of the result is the
    sequence position of the row stored at rank-major index p.
    """
    if S % (2 * N):
        raise ValueError("S must be divisible by 2N")
    c = S // (2 * N)
    order = np.empty(S, dtype=np.int64)
    p = 0
    for i in range(N):
        for chunk in (i, 2 * N - 1 - i):
            order[p:p + c] = np.arange(chunk * c, (chunk + 1) * c)
            p += c
    return order


def striped_order(S: int, N: int) -> np.ndarray:
    """Sequence positions in rank-major memory order for the striped split
    [SP "Causal Masking and Load Balancing"]: token t goes to rank t mod N, and
    each rank keeps its tokens in sequence order."""
    if S % N:
        raise ValueError("S must be divisible by N")
    order = np.empty(S, dtype=np.int64)
    p = 0
    for r in range(N):
        for t in range(S):
            if t % N == r:
                order[p] = t
                p += 1
    return order


def layout_order(S: int, N: int, layout: str) -> np.ndarray:
    if layout == "contiguous":
        return contiguous_order(S, N)
    if layout == "zigzag":
        return zigzag_order(S, N)
    if layout == "striped":
        return striped_order(S, N)
    raise ValueError(f"unknown layout {layout!r}")


def rank_positions(S: int, N: int, layout: str, rank: int) -> np.ndarray:
    """Global positions of the C = S/N rows rank ``rank`` holds, in memory order."""
    C = S // N
    return layout_order(S, N, layout)[rank * C:(rank + 1) * C]


def permute_rows(x, order: np.ndarray, axis: int = -2):
    """Gather rows of ``x`` along ``axis`` into rank-major order."""
    return np.take(np.asarray(x), order, axis=axis)


def unpermute_rows(x, order: np.ndarray, axis: int = -2):
    """Inverse of ``permute_rows``: rank-major order back to sequence order."""
    x = np.asarray(x)
    out = np.empty_like(x)
    idx = [slice(None)] * x.ndim
    idx[axis] = order
    out[tuple(idx)] = x
    return out


# ---------------------------------------------------------------------------
# Ring schedule [SP "Algorithmic Mechanics" item 2; the 4-GPU figure;
# CP listing: source=(rank - step) % world].
# ---------------------------------------------------------------------------
def ring_source(rank: int, step: int, N: int) -> int:
    """Rank whose KV block device ``rank`` holds at ring step ``step``."""
    return (rank - step) % N


def ring_schedule(N: int) -> np.ndarray:
    """[rank, step] -> source rank of the KV block used at that step."""
    return np.array([[ring_source(r, s, N) for s in range(N)]
                     for r in range(N)], dtype=np.int64)


# ---------------------------------------------------------------------------
# Online-softmax merge [SP "Algorithmic Mechanics", m_new / l_new / O_new].
# ---------------------------------------------------------------------------
def _online_softmax_update(m_prev, l_prev, O_prev, m_blk, l_blk, O_blk_sum):
    """One application of the pages' running-statistics update.

    m_prev, l_prev, O_prev: running max, running sum of exponentials and the
    normalised running output. m_blk, l_blk: the block's row max and sum of
    exp(s - m_blk); O_blk_sum: the UNNORMALISED block output
    sum_j exp(s_j - m_blk) v_j. Rows where both maxima are -inf stay empty.
    """
    m_new = np.maximum(m_prev, m_blk)
    ok = m_new > NEG_INF
    m_ref = np.where(ok, m_new, 0.0)
    a = np.where(m_prev > NEG_INF, np.exp(m_prev - m_ref), 0.0)
    b = np.where(m_blk > NEG_INF, np.exp(m_blk - m_ref), 0.0)
    l_new = l_prev * a + l_blk * b
    den = np.where(ok, l_new, 1.0)
    O_new = (O_prev * (l_prev * a / den)[..., None]
             + O_blk_sum * (b / den)[..., None])
    return m_new, l_new, O_new


def merge(out_a, lse_a, out_b, lse_b):
    """Merge two normalised partial results (out, lse) over disjoint key sets.

    Each partial is written in the pages' (m, l, O) form with m = lse and
    l = 1, so l * exp(m) = exp(lse), and its unnormalised block sum is
    l * out. Returns (out, lse) of attention over the union of the key sets.
    """
    out_a, lse_a = to_f64(out_a), to_f64(lse_a)
    out_b, lse_b = to_f64(out_b), to_f64(lse_b)
    l_a = np.where(lse_a > NEG_INF, 1.0, 0.0)
    l_b = np.where(lse_b > NEG_INF, 1.0, 0.0)
    m_new, l_new, O_new = _online_softmax_update(
        lse_a, l_a, out_a, lse_b, l_b, out_b * l_b[..., None])
    lse = np.where(l_new > 0, m_new + np.log(np.where(l_new > 0, l_new, 1.0)),
                   NEG_INF)
    return O_new, lse


# ---------------------------------------------------------------------------
# The ring itself, in float64 [CP listing and "Ring attention"; SP
# "Algorithmic Mechanics"]. It is a second, independent route to the same
# result as ``attention`` and is used to pin the exactness statement.
# ---------------------------------------------------------------------------
def ring_attention(q, k, v, *, N: int, layout: str, causal: bool,
                   scale: float | None = None, kv_head_of_q=None):
    """Simulate the N-rank ring in float64 and return (out, lse) in sequence order.

    Rank r keeps its query block and starts from out = 0, m = -inf, l = 0. At
    step t = 0..N-1 it holds the KV block of source (r - t) mod N, computes the
    block's masked scores against its queries using GLOBAL positions, and folds
    them into the running statistics with the online-softmax update.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kv_map = _kv_map(Hq, Hkv, kv_head_of_q)
    order = layout_order(S, N, layout)
    C = S // N
    out = np.zeros((B, Hq, S, D))
    lse = np.full((B, Hq, S), NEG_INF)
    for r in range(N):
        q_rows = order[r * C:(r + 1) * C]
        for b in range(B):
            for h in range(Hq):
                g = kv_map[h]
                qr = q[b, h, q_rows]
                m = np.full(C, NEG_INF)
                l = np.zeros(C)
                O = np.zeros((C, D))
                for step in range(N):
                    src = ring_source(r, step, N)
                    k_rows = order[src * C:(src + 1) * C]
                    s = scale * (qr @ k[b, g, k_rows].T)
                    if causal:
                        s = np.where(k_rows[None, :] <= q_rows[:, None], s,
                                     NEG_INF)
                    m_blk = s.max(axis=1)
                    p = np.zeros_like(s)
                    ok = m_blk > NEG_INF
                    p[ok] = np.exp(s[ok] - m_blk[ok, None])
                    l_blk = p.sum(axis=1)
                    O_blk_sum = p @ v[b, g, k_rows]
                    m, l, O = _online_softmax_update(m, l, O, m_blk, l_blk,
                                                     O_blk_sum)
                out[b, h, q_rows] = O
                lse[b, h, q_rows] = np.where(
                    l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return out, lse


# ---------------------------------------------------------------------------
# Useful work [CP "The causal imbalance": masked-in work per rank].
# ---------------------------------------------------------------------------
def useful_pairs(q_pos, k_pos, causal: bool) -> int:
    """Number of (query, key) pairs the mask allows, by brute force."""
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.asarray(k_pos, np.int64)
    if not causal:
        return int(len(q_pos) * len(k_pos))
    return int((k_pos[None, :] <= q_pos[:, None]).sum())


def pairs_per_rank_step(S: int, N: int, layout: str, causal: bool) -> np.ndarray:
    """[rank, step] -> allowed (query, key) pairs per head, by brute force."""
    C = S // N
    order = layout_order(S, N, layout)
    out = np.zeros((N, N), dtype=np.int64)
    for r in range(N):
        qp = order[r * C:(r + 1) * C]
        for step in range(N):
            src = ring_source(r, step, N)
            out[r, step] = useful_pairs(qp, order[src * C:(src + 1) * C], causal)
    return out


def useful_flops(B: int, Hq: int, D: int, pairs_per_head: int) -> int:
    """4*D flops per allowed pair: 2*D for q.k and 2*D for p*v."""
    return 4 * D * B * Hq * int(pairs_per_head)
