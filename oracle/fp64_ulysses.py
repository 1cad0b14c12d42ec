"""Plain fp64 CPU oracle for DeepSpeed-Ulysses sequence parallelism.

TEST INFRASTRUCTURE ONLY, like ``oracle.fp64``: imported by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the HIP library.

Source (cited by page title and section):
  [SP]  "Sequence Parallelism in Large Language Models ..." (llms.blog):
        section "DeepSpeed Ulysses: Head-to-Sequence All-to-All
        Transposition" -- the layout diagram (each rank's [Batch, S/P, H, D]
        slice; an all-to-all to [Batch, S, H/P, D]; local attention on the
        full sequence; an all-to-all back), "Execution Flow" items 2-4, and
        "Communication Cost and Constraints" (the volume of one all-to-all,
        (P-1)/P * b*s*h; H divisible by P; P <= H_KV under GQA).
  [SCP] "Sequence and Context Parallelism" (praveentn.live): "What it does
        not change" -- the result equals single-device attention.

Readings taken where the pages are silent:
  * rank p's input slice is the contiguous sequence slice [p*S/P, (p+1)*S/P)
    (the pages only say each rank holds s/P of the sequence);
  * after the first all-to-all rank j holds heads [j*H/P, (j+1)*H/P) for the
    whole sequence, the slices received from ranks 0..P-1 stacked in rank
    order, so global position t is row t;
  * GQA: query heads and KV heads are both split into P contiguous groups;
    a rank's query heads must read only its own KV heads (with the default
    map h -> h // (Hq/Hkv) that holds whenever P divides Hkv);
  * the local attention is exact attention over the full sequence with
    positions 0..S-1 (the causal rule as in ``oracle.attention``);
  * the log-sum-exp stays on the rank that computed it, in the head-sharded
    layout [B, H/P, S] (the pages move only the attention output back).
"""
from __future__ import annotations

import numpy as np

from .fp64 import _kv_map, attention, to_f64


def _check(P: int, S: int, H: int) -> None:
    if P < 1 or S % P or H % P:
        raise ValueError(f"Ulysses needs S and H divisible by P (S={S}, H={H}, P={P})")


def ulysses_all_to_all(x, P: int):
    """First all-to-all [SP Ulysses, Execution Flow item 2]: sequence gather,
    head scatter. ``x`` is [P, B, S/P, H, D] (rank p's sequence slice in x[p]);
    returns [P, B, S, H/P, D]: rank j receives, from every rank p, p's slice
    for heads j*H/P .. (j+1)*H/P - 1 and places it at sequence offset p*S/P."""
    x = np.asarray(x)
    _, B, Sp, H = x.shape[:4]
    S = Sp * P
    _check(P, S, H)
    Hp = H // P
    y = np.zeros((P, B, S, Hp) + x.shape[4:], dtype=x.dtype)
    for j in range(P):           # receiving rank
        for p in range(P):       # sending rank
            y[j, :, p * Sp:(p + 1) * Sp] = x[p, :, :, j * Hp:(j + 1) * Hp]
    return y


def ulysses_all_to_all_inverse(y, P: int):
    """Second all-to-all [SP Ulysses, Execution Flow item 4]: head gather,
    sequence scatter, [P, B, S, H/P, D] -> [P, B, S/P, H, D]. Rank p receives,
    from every rank j, the rows p*S/P .. (p+1)*S/P - 1 of j's heads."""
    y = np.asarray(y)
    _, B, S, Hp = y.shape[:4]
    Sp = S // P
    _check(P, S, Hp * P)
    x = np.zeros((P, B, Sp, Hp * P) + y.shape[4:], dtype=y.dtype)
    for p in range(P):           # receiving rank
        for j in range(P):       # sending rank
            x[p, :, :, j * Hp:(j + 1) * Hp] = y[j, :, p * Sp:(p + 1) * Sp]
    return x


def ulysses_attention(q, k, v, *, P: int, causal: bool, scale: float | None = None,
                      kv_head_of_q=None):
    """Ulysses forward in float64 [SP Ulysses, Execution Flow items 2-4].

    q: [P, B, S/P, Hq, D]; k, v: [P, B, S/P, Hkv, D] (the ranks' sequence
    slices). Returns (out [P, B, S/P, Hq, D], lse [P, B, Hq/P, S]).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    Hq, Hkv = q.shape[3], k.shape[3]
    S = q.shape[2] * P
    _check(P, S, Hq)
    _check(P, S, Hkv)
    Hqp, Hkvp = Hq // P, Hkv // P
    kv_map = _kv_map(Hq, Hkv, kv_head_of_q)
    for h in range(Hq):
        if kv_map[h] // Hkvp != h // Hqp:
            raise ValueError(f"query head {h} reads KV head {kv_map[h]} held by another rank")
    qh, kh, vh = (ulysses_all_to_all(t, P) for t in (q, k, v))   # [P, B, S, H/P, D]
    outh = np.zeros_like(qh)
    lse = np.zeros((P, q.shape[1], Hqp, S))
    for j in range(P):
        local_map = [kv_map[j * Hqp + h] - j * Hkvp for h in range(Hqp)]
        # the local kernel sees [B, heads, S, D]
        o, l = attention(qh[j].transpose(0, 2, 1, 3), kh[j].transpose(0, 2, 1, 3),
                         vh[j].transpose(0, 2, 1, 3), causal=causal, scale=scale,
                         kv_head_of_q=local_map)
        outh[j] = o.transpose(0, 2, 1, 3)
        lse[j] = l
    return ulysses_all_to_all_inverse(outh, P), lse


def ulysses_volume(B: int, S: int, H: int, D: int, P: int) -> float:
    """Elements that change rank in one all-to-all [SP Ulysses, "Communication
    Cost and Constraints"]: (P-1)/P * b*s*h, h = H*D the hidden size.

    Reading: every rank keeps 1/P of its own b*(s/P)*h slice and sends the
    rest, so the formula is the sum over the P ranks (or, per rank, the same
    expression with s read as the local length s/P); the per-rank figure
    (P-1)/P * b*(s/P)*h is the one that stays constant when s and P grow
    together, as the page says."""
    return (P - 1) / P * B * S * H * D


# ---------------------------------------------------------------------------
# Unified sequence parallelism [SP "Unified Sequence Parallelism (USP / 2D
# SP)": Ulysses all-to-all inside a node across heads, the ring across nodes
# circulating (K, V)].
#
# Readings (the page gives the grid, not the token assignment):
#   * the ring dimension assigns tokens to the P_r nodes as the ring layout
#     does for P_r ranks (contiguous, zigzag or striped); node n's token list
#     L_n is that rank's positions in memory order;
#   * inside node n, device u of the P_u Ulysses devices holds the contiguous
#     piece L_n[u*C/P_u : (u+1)*C/P_u] (C = S/P_r) for all heads;
#   * the intra-node all-to-all gives device u of every node the node's whole
#     list L_n for head group u; the ring then runs over the P_r nodes, once
#     per head group, on those tokens; the reverse all-to-all returns the
#     output to the device slices;
#   * lse stays with the device that computed it: [P_u, B, H/P_u, S], its
#     sequence axis in node-major order (L_0, then L_1, ...).
# ---------------------------------------------------------------------------
def usp_token_lists(S: int, P_r: int, layout: str) -> np.ndarray:
    """[P_r, S/P_r] global positions of each node's tokens (the ring layout)."""
    from .fp64 import layout_order
    return layout_order(S, P_r, layout).reshape(P_r, S // P_r)


def usp_attention(q, k, v, *, P_u: int, P_r: int, layout: str, causal: bool,
                  scale: float | None = None, kv_head_of_q=None):
    """USP forward in float64.

    q: [P_r*P_u, B, S/(P_r*P_u), Hq, D], k, v: [.., Hkv, D]: the slice of
    device d = n*P_u + u, holding positions usp_token_lists(...)[n][u-th
    piece]. Returns (out in the same layout as q, lse [P_u, B, Hq/P_u, S]).
    """
    from .fp64 import ring_attention
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    P = P_r * P_u
    _, B, Sp, Hq, D = q.shape
    Hkv = k.shape[3]
    C = Sp * P_u                     # tokens per node
    S = C * P_r
    _check(P_u, C, Hq)
    _check(P_u, C, Hkv)
    kv_map = _kv_map(Hq, Hkv, kv_head_of_q)
    Hqp, Hkvp = Hq // P_u, Hkv // P_u
    for h in range(Hq):
        if kv_map[h] // Hkvp != h // Hqp:
            raise ValueError(f"query head {h} reads KV head {kv_map[h]} held by another device")
    lists = usp_token_lists(S, P_r, layout)
    # intra-node all-to-all: node n's devices -> [P_u, B, C, H/P_u, D]
    heads = [[ulysses_all_to_all(t[n * P_u:(n + 1) * P_u], P_u) for n in range(P_r)]
             for t in (q, k, v)]
    out_h = [np.zeros_like(heads[0][n]) for n in range(P_r)]
    lse = np.zeros((P_u, B, Hqp, S))
    order = lists.reshape(-1)        # node-major position list
    inv = np.argsort(order)
    for u in range(P_u):
        local_map = [kv_map[u * Hqp + h] - u * Hkvp for h in range(Hqp)]
        # head group u over the whole sequence, in sequence order: [B, heads, S, D]
        seq = []
        for t in range(3):
            nm = np.concatenate([heads[t][n][u] for n in range(P_r)], axis=1)  # [B, S, H, D]
            seq.append(nm.transpose(0, 2, 1, 3)[:, :, inv])
        o, l = ring_attention(seq[0], seq[1], seq[2], N=P_r, layout=layout, causal=causal,
                              scale=scale, kv_head_of_q=local_map)
        o_nm, l_nm = o[:, :, order], l[:, :, order]      # back to node-major order
        for n in range(P_r):
            out_h[n][u] = o_nm[:, :, n * C:(n + 1) * C].transpose(0, 2, 1, 3)
        lse[u] = l_nm
    out = np.concatenate([ulysses_all_to_all_inverse(out_h[n], P_u) for n in range(P_r)], axis=0)
    return out, lse
