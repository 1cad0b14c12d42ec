"""GPU parity of the backward path (through the C ABI) against the fp64 oracle.

Tolerance for bf16 inputs: every gradient element is a sum of products in
which one factor (the probability p or ds) is rounded to bf16 (up to 2^-9
relative) before an fp32 accumulation; the sums cancel strongly (sum_j ds_ij
= 0), so the error relative to the gradient's typical size is of the order
of that rounding, ~2e-3. The ring path also rounds the final gradients to
bf16 (another <= 2^-9) and uses the forward's bf16 output for delta. Errors
are judged per tensor (dq, dk, dv) relative to its scale:
  max |g - r| <= TOL_MAX * max |r|   and   mean |g - r| <= TOL_MEAN * mean |r|
with TOL_MEAN = 4e-3 (the two roundings) and TOL_MAX = 1e-2.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_context_parallelism_flash_amd")
DEV = "cuda"
TOL_MAX = 1e-2
TOL_MEAN = 4e-3


def _rnd(shape, seed, dtype=torch.bfloat16, scale=1.0):
    return workloads.make_random(shape, seed, dtype, scale)


def _pos_array(desc, rows):
    if desc is None:
        return np.arange(rows)
    nseg, seg, *rest = desc
    rest = list(rest) + [0] * (3 - len(rest))
    s0, s1, stride = rest[0], rest[1], rest[2] or 1
    t = np.arange(rows)
    if nseg == 1:
        return s0 + t * stride
    return np.where(t < seg, s0 + t * stride, s1 + (t - seg) * stride)


def _np(t):
    return t.detach().double().cpu().numpy()


def _check_grads(got, ref, what):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        scale_max = max(np.abs(r).max(), 1e-30)
        scale_mean = max(np.abs(r).mean(), 1e-30)
        e_max = np.abs(g - r).max() / scale_max
        e_mean = np.abs(g - r).mean() / scale_mean
        print(f"{what} {name}: rel max {e_max:.2e} rel mean {e_mean:.2e}", flush=True)
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        assert e_max <= TOL_MAX, f"{what} {name}: max err {e_max:.3e} > {TOL_MAX}"
        assert e_mean <= TOL_MEAN, f"{what} {name}: mean err {e_mean:.3e} > {TOL_MEAN}"


# ---------------------------------------------------------------- block
BLOCK_CASES = [
    # Cq, Ck, q_pos, k_pos, causal, Hq, Hkv, D
    (128, 128, None, None, True, 2, 2, 128),
    (300, 200, None, None, True, 4, 2, 128),                       # ragged tiles, GQA
    (257, 513, (1, 257, 1000), None, True, 2, 1, 64),              # all keys visible
    (384, 320, (2, 192, 100, 700), (2, 160, 0, 600), True, 2, 2, 128),
    (256, 256, (1, 256, 1, 0, 4), (1, 256, 2, 0, 4), True, 2, 2, 128),   # striped ranks
    (200, 333, None, None, False, 4, 1, 64),
    (5, 3, (1, 5, 2), None, True, 2, 2, 128),
    (130, 70, (1, 130, 0, 0, 7), (1, 70, 5, 0, 7), False, 2, 2, 64),
    (64, 96, (1, 64, 0), (1, 96, 40), True, 2, 2, 128),            # rows 0..39 see no key
    (256, 256, None, None, True, 2, 1, 64),    # D=64 diagonal: mask-free and masked sub-tiles
    (192, 192, None, None, True, 1, 1, 64),
    # D=128 blocks of whole 64-key tiles (the one-wave-per-SIMD dq kernel)
    (300, 192, None, None, True, 4, 2, 128),                       # ragged query rows
    (384, 128, (1, 384, 0), (1, 128, 200), True, 8, 2, 128),       # keys inside the rows' span
    (96, 512, (1, 96, 500), None, False, 2, 2, 128),               # non-causal, few rows
]


@pytest.mark.parametrize("case", range(len(BLOCK_CASES)))
def test_block_bwd_vs_oracle(case):
    Cq, Ck, qp, kp, causal, Hq, Hkv, D = BLOCK_CASES[case]
    seed = 100 + 10 * case
    q, k, v = _rnd((1, Hq, Cq, D), seed), _rnd((1, Hkv, Ck, D), seed + 1), _rnd((1, Hkv, Ck, D), seed + 2)
    dout = _rnd((1, Hq, Cq, D), seed + 3)
    qpa, kpa = _pos_array(qp, Cq), _pos_array(kp, Ck)
    out, lse = oracle.attention(q, k, v, causal=causal, q_pos=qpa, k_pos=kpa)
    ref = oracle.attention_backward(q, k, v, dout, causal=causal, q_pos=qpa, k_pos=kpa)
    out_t = torch.from_numpy(out).to(torch.bfloat16)
    lse_t = torch.from_numpy(lse).float()
    dq = torch.zeros(1, Hq, Cq, D, device=DEV)
    dk = torch.zeros(1, Hkv, Ck, D, device=DEV)
    dv = torch.zeros(1, Hkv, Ck, D, device=DEV)
    ra.ra_block_attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), out_t.to(DEV), dout.to(DEV),
                         lse_t.to(DEV), dq, dk, dv, q_pos=qp, k_pos=kp, causal=causal)
    torch.cuda.synchronize()
    _check_grads([_np(dq), _np(dk), _np(dv)], ref, f"block case {case}")


def test_block_bwd_accumulates_bitexact():
    """Two identical calls add the same values twice: the result is exactly 2x."""
    Cq = Ck = 192
    q, k, v = _rnd((1, 2, Cq, 128), 1), _rnd((1, 2, Ck, 128), 2), _rnd((1, 2, Ck, 128), 3)
    dout = _rnd((1, 2, Cq, 128), 4)
    out, lse = oracle.attention(q, k, v, causal=True)
    args = [t.to(DEV) for t in (q, k, v, torch.from_numpy(out).to(torch.bfloat16), dout,
                                torch.from_numpy(lse).float())]
    grads = [torch.zeros(1, 2, Cq, 128, device=DEV) for _ in range(3)]
    ra.ra_block_attn_bwd(*args, *grads, causal=True)
    once = [g.clone() for g in grads]
    ra.ra_block_attn_bwd(*args, *grads, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(grads, once):
        assert torch.equal(a, 2 * b)


# ---------------------------------------------------------------- ring
RINGS = [
    workloads.Workload("bwd_zigzag_gqa", B=1, Hq=4, Hkv=2, D=128, S=1024, dtype="bf16", seed=51,
                       causal=True, N=4, layout="zigzag"),
    workloads.Workload("bwd_contig_d64", B=2, Hq=2, Hkv=1, D=64, S=768, dtype="bf16", seed=52,
                       causal=True, N=3, layout="contiguous"),
    workloads.Workload("bwd_striped_ragged", B=1, Hq=2, Hkv=2, D=128, S=1000, dtype="bf16",
                       seed=53, causal=True, N=8, layout="striped"),
    workloads.Workload("bwd_noncausal", B=1, Hq=2, Hkv=1, D=128, S=512, dtype="bf16", seed=54,
                       causal=False, N=4, layout="contiguous"),
    workloads.Workload("bwd_single_rank", B=1, Hq=2, Hkv=2, D=128, S=640, dtype="bf16", seed=55,
                       causal=True, N=1, layout="zigzag"),
    # five query heads per KV head, five ranks, 101-token chunks (ragged tiles)
    workloads.Workload("bwd_zigzag_gqa5_n5_ragged", B=1, Hq=5, Hkv=1, D=64, S=1010,
                       dtype="bf16", seed=56, causal=True, N=5, layout="zigzag"),
    # non-causal zigzag with two batches
    workloads.Workload("bwd_noncausal_zigzag_b2", B=2, Hq=4, Hkv=2, D=64, S=600, dtype="bf16",
                       seed=57, causal=False, N=3, layout="zigzag"),
]


def _ring_fwd_bwd(w, dout_seed):
    q, k, v = workloads.make_inputs(w)
    dout = _rnd(q.shape, dout_seed)
    qd, kd, vd, dd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ra.ring_attention_sim(qd, kd, vd, N=w.N, layout=w.layout, causal=w.causal)
    dq, dk, dv = ra.ring_attention_sim_backward(qd, kd, vd, out, lse, dd, N=w.N,
                                                layout=w.layout, causal=w.causal)
    torch.cuda.synchronize()
    return (q, k, v, dout), (dq, dk, dv)


@pytest.mark.parametrize("w", RINGS, ids=[w.name for w in RINGS])
def test_ring_bwd_vs_oracle(w):
    (q, k, v, dout), got = _ring_fwd_bwd(w, w.seed + 100)
    ref = oracle.attention_backward(q, k, v, dout, causal=w.causal)
    _check_grads([_np(t) for t in got], ref, f"ring {w.name}")


def test_ring_bwd_gqa_128k_rows_suffix_and_invariants():
    """At the 128k GQA zigzag shape, element by element against the oracle:
    dq on 64 seeded rows per head plus fixed rows (both ends of the sequence
    and of the first chunk, the middle), and dk, dv of the last 256 key
    positions of every KV head. Under the causal rule only the queries at or
    after a key see it, so those keys' gradients need just the last 256 query
    rows of the group's heads, which are among the rows. Over all rows, sum_j
    dv_j equals the group's sum_i dout_i and sum_j dk_j vanishes."""
    from parity_util import pooled_backward
    w = workloads.HEADLINE
    (q, k, v, dout), (dq, dk, dv) = _ring_fwd_bwd(w, 977)
    n = int(os.environ.get("RA_ORACLE_ROWS_BWD", "64"))
    L = 256
    c = w.S // (2 * w.N)
    fixed = np.union1d(np.array([0, c - 1, c, w.S // 2]), np.arange(w.S - L, w.S))
    rest = np.setdiff1d(np.arange(w.S), fixed)
    rows = np.stack([np.sort(np.concatenate(
        [fixed, np.random.default_rng([w.seed, h]).choice(rest, n, replace=False)]))
        for h in range(w.Hq)])
    print(f"128k backward: dq on {rows.shape[1]} rows per head x {w.Hq} heads; dk, dv on the "
          f"last {L} keys of {w.Hkv} KV heads", flush=True)
    ref_dq, ref_dk, ref_dv = pooled_backward(q, k, v, dout, rows=rows, key0=w.S - L)
    got_dq = np.stack([_np(dq[0, h, torch.from_numpy(rows[h])]) for h in range(w.Hq)])
    got_dk = _np(dk[0, :, w.S - L:])
    got_dv = _np(dv[0, :, w.S - L:])
    _check_grads([got_dq, got_dk, got_dv], [ref_dq, ref_dk, ref_dv], "128k rows / key suffix")
    group = w.Hq // w.Hkv
    dsum = dout.double().view(1, w.Hkv, group, w.S, w.D).sum(dim=(2, 3))[0]
    dv_sum = dv.double().sum(dim=2)[0].cpu()
    dk_sum = dk.double().sum(dim=2)[0].cpu()
    dk_abs = dk.double().abs().sum(dim=2)[0].cpu()
    e_dv = ((dv_sum - dsum).abs().max() / dsum.abs().max()).item()
    e_dk = (dk_sum.abs() / dk_abs).max().item()
    print(f"128k invariants: sum dv vs sum dout rel {e_dv:.2e}; |sum dk| / sum |dk| {e_dk:.2e}",
          flush=True)
    assert e_dv <= 1e-2
    assert e_dk <= 1e-3


# ------------------------------------------------------- head maps and groups
@pytest.mark.parametrize("kv_map,Hkv", [
    ([1, 0, 1, 0, 0, 1], 2),
    ([2, 0, 1, 1, 2, 0, 0, 2], 3),
    # 66 query heads on KV head 0: more than a wave's 64 lanes can hold, so
    # the dk/dv kernel reads the group's heads from its LDS table
    ([1 if i % 12 == 0 else 0 for i in range(72)], 2),
], ids=["6q_2kv", "8q_3kv", "72q_group66"])
def test_block_bwd_custom_head_map(kv_map, Hkv):
    """Query heads that read their KV heads out of order (the dk/dv kernel
    walks each KV head's query heads from a per-workgroup head list: one head
    per lane for groups of up to 64, an LDS table beyond)."""
    Hq, Cq, Ck, D = len(kv_map), 192, 160, 128
    q, k, v = _rnd((1, Hq, Cq, D), 71), _rnd((1, Hkv, Ck, D), 72), _rnd((1, Hkv, Ck, D), 73)
    dout = _rnd((1, Hq, Cq, D), 74)
    qp, kp = (1, Cq, 100), (1, Ck, 0)
    qpa, kpa = _pos_array(qp, Cq), _pos_array(kp, Ck)
    out, lse = oracle.attention(q, k, v, causal=True, q_pos=qpa, k_pos=kpa, kv_head_of_q=kv_map)
    ref = oracle.attention_backward(q, k, v, dout, causal=True, q_pos=qpa, k_pos=kpa,
                                    kv_head_of_q=kv_map)
    dq = torch.zeros(1, Hq, Cq, D, device=DEV)
    dk = torch.zeros(1, Hkv, Ck, D, device=DEV)
    dv = torch.zeros(1, Hkv, Ck, D, device=DEV)
    ra.ra_block_attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(out).to(torch.bfloat16).to(DEV),
                         dout.to(DEV), torch.from_numpy(lse).float().to(DEV), dq, dk, dv,
                         q_pos=qp, k_pos=kp, causal=True, kv_head_of_q=kv_map)
    torch.cuda.synchronize()
    _check_grads([_np(dq), _np(dk), _np(dv)], ref, f"head map {kv_map}")


def test_ring_bwd_large_group_and_map():
    """16 query heads on one KV head (one long head stream per workgroup) and a
    ring with a permuted head map."""
    w = workloads.Workload("bwd_mqa16", B=1, Hq=16, Hkv=1, D=64, S=512, dtype="bf16", seed=81,
                           causal=True, N=4, layout="zigzag")
    (q, k, v, dout), got = _ring_fwd_bwd(w, 181)
    _check_grads([_np(t) for t in got], oracle.attention_backward(q, k, v, dout, causal=True),
                 "ring mqa16")
    kv_map = [1, 1, 0, 1, 0, 0]
    q, k, v = _rnd((1, 6, 384, 128), 82), _rnd((1, 2, 384, 128), 83), _rnd((1, 2, 384, 128), 84)
    dout = _rnd((1, 6, 384, 128), 85)
    qd, kd, vd, dd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ra.ring_attention_sim(qd, kd, vd, N=3, layout="striped", causal=True,
                                     kv_head_of_q=kv_map)
    grads = ra.ring_attention_sim_backward(qd, kd, vd, out, lse, dd, N=3, layout="striped",
                                           causal=True, kv_head_of_q=kv_map)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(q, k, v, dout, causal=True, kv_head_of_q=kv_map)
    _check_grads([_np(t) for t in grads], ref, "ring striped head map")
