"""Plain fp64 CPU oracle for the ring-attention BACKWARD step.

TEST INFRASTRUCTURE ONLY, like ``oracle.fp64``: imported by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the HIP library.

Sources (cited by page title and section):
  [SCP] "Sequence and Context Parallelism" (praveentn.live): section "What it
        does not change" -- the loss and the gradients under context
        parallelism are those of single-device attention.
  [SP]  "Sequence Parallelism in Large Language Models ..." (llms.blog):
        section "The Activation Memory Wall in Long-Context Scaling" (the
        attention probabilities are recomputed in the backward pass rather
        than stored) and "Algorithmic Mechanics" (the ring: at step t rank r
        holds the KV block of source (r - t) mod P).

The pages give no backward algorithm. Readings taken:
  * the definition is the derivative of exact softmax attention (the
    forward's definition in ``oracle.fp64``): with p_ij = exp(s_ij - lse_i) on
    allowed pairs, s_ij = scale * <q_i, k_j>, out_i = sum_j p_ij v_j and an
    upstream gradient dout,
        dv_j  = sum_i p_ij dout_i
        dp_ij = <dout_i, v_j>
        delta_i = <dout_i, out_i>          (= sum_j p_ij dp_ij)
        ds_ij = p_ij (dp_ij - delta_i)
        dq_i  = scale * sum_j ds_ij k_j
        dk_j  = scale * sum_i ds_ij q_i
    with GQA gradients of a KV head summed over the query heads that read it;
    a row with no allowed key contributes nothing;
  * the ring backward mirrors the forward ring: rank r keeps its q, dout, lse
    and delta; at step t it holds the KV block of source (r - t) mod N,
    recomputes that block's probabilities from the FINAL lse, adds its dq
    contribution at home and the block's dk, dv contributions to source
    (r - t) mod N (in a real ring they travel with the block).
"""
from __future__ import annotations

import math

import numpy as np

from .fp64 import NEG_INF, _kv_map, layout_order, ring_source, to_f64


def attention_backward(q, k, v, dout, *, causal: bool, scale: float | None = None,
                       kv_head_of_q=None, q_pos=None, k_pos=None):
    """Gradients (dq, dk, dv) of exact softmax attention, float64.

    Shapes as in ``oracle.attention``: q, dout [B, Hq, Sq, D]; k, v
    [B, Hkv, Sk, D]. Positions and the causal rule as there.
    """
    q, k, v, dout = to_f64(q), to_f64(k), to_f64(v), to_f64(dout)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kv_map = _kv_map(Hq, Hkv, kv_head_of_q)
    q_pos = np.arange(Sq) if q_pos is None else np.asarray(q_pos, np.int64)
    k_pos = np.arange(Sk) if k_pos is None else np.asarray(k_pos, np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = kv_map[h]
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s = np.where(k_pos[None, :] <= q_pos[:, None], s, NEG_INF)
            m = s.max(axis=1)
            ok = m > NEG_INF
            p = np.zeros_like(s)
            p[ok] = np.exp(s[ok] - m[ok, None])
            p[ok] /= p[ok].sum(axis=1, keepdims=True)
            out = p @ v[b, g]
            dp = dout[b, h] @ v[b, g].T
            delta = (dout[b, h] * out).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
            dv[b, g] += p.T @ dout[b, h]
    return dq, dk, dv


def attention_backward_dq_rows(q, k, v, dout, rows, *, causal: bool, scale: float | None = None,
                                kv_head_of_q=None):
    """dq of selected query rows only, float64 (the same definition as
    ``attention_backward``; each dq row needs only its own row's scores).
    ``rows`` is [Hq, R] per-head row indices; returns [B, Hq, R, D]."""
    q, k, v, dout = to_f64(q), to_f64(k), to_f64(v), to_f64(dout)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kv_map = _kv_map(Hq, Hkv, kv_head_of_q)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((B, Hq, rows.shape[1], D))
    for b in range(B):
        for h in range(Hq):
            g = kv_map[h]
            for r, i in enumerate(rows[h]):
                kk = k[b, g, :i + 1] if causal else k[b, g]
                vv = v[b, g, :i + 1] if causal else v[b, g]
                s = scale * (kk @ q[b, h, i])
                p = np.exp(s - s.max())
                p /= p.sum()
                out = p @ vv
                dp = vv @ dout[b, h, i]
                ds = p * (dp - dout[b, h, i] @ out)
                dq[b, h, r] = scale * (ds @ kk)
    return dq


def block_backward(q, k, v, dout, lse, delta, *, causal: bool, scale: float,
                   q_pos, k_pos):
    """One block pair's gradient contributions for one head, float64.

    q, dout: [Cq, D]; k, v: [Ck, D]; lse, delta: [Cq] (from the whole
    forward). Returns (dq [Cq, D], dk [Ck, D], dv [Ck, D]).
    """
    s = scale * (q @ k.T)
    allowed = np.ones(s.shape, dtype=bool)
    if causal:
        allowed = k_pos[None, :] <= q_pos[:, None]
    finite = lse > NEG_INF
    p = np.zeros_like(s)
    use = allowed & finite[:, None]
    p[use] = np.exp(s - np.where(finite, lse, 0.0)[:, None])[use]
    dp = dout @ v.T
    ds = p * (dp - delta[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), p.T @ dout


def ring_attention_backward(q, k, v, dout, out, lse, *, N: int, layout: str, causal: bool,
                            scale: float | None = None, kv_head_of_q=None):
    """The N-rank ring backward in float64, inputs and results in sequence order.

    ``out`` and ``lse`` are the forward results (sequence order). Rank r
    computes delta = <dout, out> for its rows once, then for t = 0..N-1 takes
    the block of source (r - t) mod N and adds that block's contributions.
    """
    q, k, v, dout = to_f64(q), to_f64(k), to_f64(v), to_f64(dout)
    out, lse = to_f64(out), to_f64(lse)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kv_map = _kv_map(Hq, Hkv, kv_head_of_q)
    order = layout_order(S, N, layout)
    C = S // N
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(N):
        q_rows = order[r * C:(r + 1) * C]
        for b in range(B):
            for h in range(Hq):
                g = kv_map[h]
                delta = (dout[b, h, q_rows] * out[b, h, q_rows]).sum(axis=1)
                for step in range(N):
                    src = ring_source(r, step, N)
                    k_rows = order[src * C:(src + 1) * C]
                    dq_b, dk_b, dv_b = block_backward(
                        q[b, h, q_rows], k[b, g, k_rows], v[b, g, k_rows], dout[b, h, q_rows],
                        lse[b, h, q_rows], delta, causal=causal, scale=scale,
                        q_pos=q_rows, k_pos=k_rows)
                    dq[b, h, q_rows] += dq_b
                    dk[b, g, k_rows] += dk_b
                    dv[b, g, k_rows] += dv_b
    return dq, dk, dv


def backward_flops(B: int, Hq: int, D: int, pairs_per_head: int) -> int:
    """Useful backward work: 10*D flops per allowed pair -- the score product
    recomputed (2D) and the four gradient products dv, dp, dq, dk (2D each)."""
    return 10 * D * B * Hq * pairs_per_head
