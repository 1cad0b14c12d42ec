"""GPU parity of the Ulysses path (through the C ABI) against the fp64 oracle.

The all-to-all is checked bit-exact against ``oracle.ulysses_all_to_all``;
the library's head-sharded layout is the oracle's [P, B, S, H/P, row] with
the local sequence and head axes swapped, so the test swaps them before
comparing. The attention is checked against ``oracle.ulysses_attention`` on
small cases (every row) and, at the 128k GQA shape, against the oracle's
exact attention on seeded rows (the Ulysses oracle equals single-device
attention; that is pinned on the CPU). Tolerances as for the ring forward.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL_BF16, TOL_F32, check_rows, compare, pooled_attention

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_context_parallelism_flash_amd")
DEV = "cuda"


def _np(t):
    return t.detach().double().cpu().numpy()


def _shard(x, P):
    """[B, H, S, D] in sequence order -> the ranks' slices [P, B, S/P, H, D]."""
    B, H, S, D = x.shape
    return x.permute(0, 2, 1, 3).reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4).contiguous()


def _unshard(x):
    """[P, B, S/P, H, D] -> [B, H, S, D]."""
    P, B, Sp, H, D = x.shape
    return x.permute(1, 0, 2, 3, 4).reshape(B, P * Sp, H, D).permute(0, 2, 1, 3)


# ---------------------------------------------------------------- all-to-all
A2A_CASES = [
    # P, B, S, H, row shape, dtype
    (2, 1, 4, 4, (8,), torch.bfloat16),
    (8, 1, 1024, 8, (128,), torch.bfloat16),     # 256-byte rows
    (4, 2, 1000, 8, (64,), torch.bfloat16),      # ragged rank slices
    (4, 1, 512, 4, (128,), torch.float32),       # 512-byte rows
    (2, 3, 64, 6, (), torch.float32),            # 4-byte rows (an lse-like array)
    (4, 1, 96, 8, (3,), torch.bfloat16),         # 6-byte rows: 2-byte accesses
    (2, 1, 16, 2, (2048,), torch.float32),       # 8 KiB rows: strided copy loop
    (1, 2, 40, 3, (16,), torch.bfloat16),        # P = 1
    # the tiled form takes T positions x all heads per workgroup, T the largest
    # power of two dividing S/P whose tile fits 64 KiB:
    (3, 1, 999, 6, (128,), torch.bfloat16),      # S/P = 333 is odd: T = 1
    (2, 1, 64, 512, (128,), torch.bfloat16),     # one position of 512 heads is 128 KiB: T = 1
    (8, 1, 64, 1032, (64,), torch.bfloat16),     # more than 1024 heads: the row gather
]


@pytest.mark.parametrize("case", range(len(A2A_CASES)))
def test_all_to_all_bitexact(case):
    P, B, S, H, row, dt = A2A_CASES[case]
    x = workloads.make_random((P, B, S // P, H) + row, 500 + case, dt)
    xd = x.to(DEV)
    y = torch.empty((P, B, H // P, S) + row, dtype=dt, device=DEV)
    ra.ra_ulysses_all_to_all(xd, y, P)
    back = torch.empty_like(xd)
    ra.ra_ulysses_all_to_all(y, back, P, inverse=True)
    torch.cuda.synchronize()
    ref = oracle.ulysses_all_to_all(x.view(torch.int16 if dt == torch.bfloat16 else torch.int32)
                                    .numpy(), P)                       # [P, B, S, H/P, row]
    got = y.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.int32).numpy()
    np.testing.assert_array_equal(np.swapaxes(got, 2, 3), ref)
    assert torch.equal(back.cpu(), x)


# ---------------------------------------------------------------- attention
SMALL = [
    # name, P, B, Hq, Hkv, S, D, dtype, causal, kv map
    ("gqa_p2", 2, 1, 4, 2, 512, 128, "bf16", True, None),
    ("ragged_b2_d64_p4", 4, 2, 8, 4, 1000, 64, "bf16", True, None),
    ("f32_mha_p4", 4, 1, 4, 4, 768, 128, "f32", True, None),
    ("noncausal_p2", 2, 1, 4, 2, 384, 128, "bf16", False, None),
    ("single_rank", 1, 1, 2, 1, 300, 128, "bf16", True, None),
    ("rank_local_map", 2, 1, 8, 4, 512, 128, "bf16", True, [1, 0, 1, 0, 3, 2, 2, 3]),
    ("p8_one_kv_head_each", 8, 1, 16, 8, 2048, 128, "bf16", True, None),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_ulysses_small_vs_oracle(case):
    name, P, B, Hq, Hkv, S, D, dt, causal, kv_map = case
    w = workloads.Workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, dtype=dt, seed=600 + len(name),
                           causal=causal, N=P, layout="ulysses")
    q, k, v = (_shard(t, P) for t in workloads.make_inputs(w))
    out = torch.empty(q.shape, dtype=q.dtype, device=DEV)
    lse = torch.empty((P, B, Hq // P, S), dtype=torch.float32, device=DEV)
    ra.ra_ulysses_sim_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, P=P, causal=causal,
                          kv_head_of_q=kv_map)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.ulysses_attention(q, k, v, P=P, causal=causal, kv_head_of_q=kv_map)
    compare(_np(out), _np(lse), ref_out, ref_lse, TOL_F32 if dt == "f32" else TOL_BF16,
            f"ulysses {name}")


def test_ulysses_repeat_bitexact():
    """Two calls on the same inputs give identical bits (no ordering effects)."""
    w = workloads.Workload("rep", B=1, Hq=8, Hkv=4, D=128, S=1024, dtype="bf16", seed=77,
                           causal=True, N=4, layout="ulysses")
    q, k, v = (_shard(t, 4).to(DEV) for t in workloads.make_inputs(w))
    outs = []
    for _ in range(2):
        out = torch.empty_like(q)
        lse = torch.empty((4, 1, 2, 1024), dtype=torch.float32, device=DEV)
        ra.ra_ulysses_sim_fwd(q, k, v, out, lse, P=4)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_ulysses_gqa_128k_sampled():
    """The 128k GQA causal inputs with 8 ranks (one KV head each): seeded rows
    plus every rank's first and last rows, against exact attention."""
    import os
    w = workloads.ULYSSES_128K
    P = w.N
    q, k, v = workloads.make_inputs(w)
    qs, ks, vs = (_shard(t, P).to(DEV) for t in (q, k, v))
    out = torch.empty(qs.shape, dtype=qs.dtype, device=DEV)
    lse = torch.empty((P, 1, w.Hq // P, w.S), dtype=torch.float32, device=DEV)
    ra.ra_ulysses_sim_fwd(qs, ks, vs, out, lse, P=P, causal=True)
    torch.cuda.synchronize()
    del qs, ks, vs
    n = int(os.environ.get("RA_ORACLE_ROWS", "32"))
    rows = check_rows(w.S, w.Hq, n, w.seed, P)
    ref_out, ref_lse = pooled_attention(q, k, v, causal=True, rows=rows)
    o = _unshard(out.cpu())[0]                                   # [Hq, S, D]
    l_ = lse.cpu()[:, 0].reshape(w.Hq, w.S)                      # rank j holds heads j*Hq/P ..
    idx = torch.from_numpy(rows)
    got_out = np.stack([o[h, idx[h]].double().numpy() for h in range(w.Hq)])
    got_lse = np.stack([l_[h, idx[h]].double().numpy() for h in range(w.Hq)])
    compare(got_out, got_lse, ref_out, ref_lse, TOL_BF16, "ulysses 128k gqa")


# ====================================================================== USP
def _usp_shard(x, P_u, P_r, layout):
    """[B, H, S, D] sequence order -> device slices [P_r*P_u, B, S/(P_r*P_u), H, D]."""
    B, H, S, D = x.shape
    L = torch.from_numpy(oracle.usp_token_lists(S, P_r, layout).reshape(-1))
    xs = x[:, :, L].permute(0, 2, 1, 3)
    return xs.reshape(B, P_r * P_u, S // (P_r * P_u), H, D).permute(1, 0, 2, 3, 4).contiguous()


USP_SMALL = [
    # name, P_u, P_r, ring layout, B, Hq, Hkv, S, D, dtype, causal, kv map
    ("usp_2x4_zigzag", 2, 4, "zigzag", 1, 4, 2, 1024, 128, "bf16", True, None),
    ("usp_2x2_striped_b2_d64", 2, 2, "striped", 2, 4, 2, 768, 64, "bf16", True, None),
    ("usp_4x2_contig_f32", 4, 2, "contiguous", 1, 4, 4, 512, 128, "f32", True, None),
    ("usp_2x2_noncausal", 2, 2, "zigzag", 1, 4, 2, 512, 128, "bf16", False, None),
    ("usp_1x4_is_ring", 1, 4, "zigzag", 1, 2, 1, 1024, 128, "bf16", True, None),
    ("usp_4x1_is_ulysses", 4, 1, "contiguous", 1, 8, 4, 512, 128, "bf16", True, None),
    ("usp_2x2_head_map", 2, 2, "zigzag", 1, 8, 4, 512, 128, "bf16", True, [1, 0, 1, 0, 3, 2, 2, 3]),
]


@pytest.mark.parametrize("case", USP_SMALL, ids=[c[0] for c in USP_SMALL])
def test_usp_small_vs_oracle(case):
    name, P_u, P_r, lay, B, Hq, Hkv, S, D, dt, causal, kv_map = case
    w = workloads.Workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, dtype=dt, seed=700 + len(name),
                           causal=causal, N=P_u * P_r, layout="usp", P_u=P_u, ring_layout=lay)
    q, k, v = (_usp_shard(t, P_u, P_r, lay) for t in workloads.make_inputs(w))
    out = torch.empty(q.shape, dtype=q.dtype, device=DEV)
    lse = torch.empty((P_u, B, Hq // P_u, S), dtype=torch.float32, device=DEV)
    ra.ra_usp_sim_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, lse, P_u=P_u, P_r=P_r, layout=lay,
                      causal=causal, kv_head_of_q=kv_map)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.usp_attention(q, k, v, P_u=P_u, P_r=P_r, layout=lay, causal=causal,
                                            kv_head_of_q=kv_map)
    compare(_np(out), _np(lse), ref_out, ref_lse, TOL_F32 if dt == "f32" else TOL_BF16,
            f"usp {name}")


def test_usp_gqa_128k_sampled():
    """The 128k GQA causal inputs on 4 nodes x 8 devices (zigzag ring across
    nodes): seeded rows plus every node's first and last positions against
    exact attention."""
    import os
    w = workloads.USP_128K
    P_u, P_r = w.P_u, w.N // w.P_u
    q, k, v = workloads.make_inputs(w)
    qs, ks, vs = (_usp_shard(t, P_u, P_r, w.ring_layout).to(DEV) for t in (q, k, v))
    out = torch.empty(qs.shape, dtype=qs.dtype, device=DEV)
    lse = torch.empty((P_u, 1, w.Hq // P_u, w.S), dtype=torch.float32, device=DEV)
    ra.ra_usp_sim_fwd(qs, ks, vs, out, lse, P_u=P_u, P_r=P_r, layout=w.ring_layout, causal=True)
    torch.cuda.synchronize()
    del qs, ks, vs
    L = oracle.usp_token_lists(w.S, P_r, w.ring_layout).reshape(-1)     # node-major positions
    inv = torch.from_numpy(np.argsort(L))
    n = int(os.environ.get("RA_ORACLE_ROWS", "32"))
    rows = check_rows(w.S, w.Hq, n, w.seed, 2 * P_r)
    ref_out, ref_lse = pooled_attention(q, k, v, causal=True, rows=rows)
    # device slices -> node-major -> sequence order
    o = out.cpu().permute(1, 0, 2, 3, 4).reshape(1, w.S, w.Hq, w.D)[0][inv]   # [S, Hq, D]
    l_ = lse.cpu()[:, 0].reshape(w.Hq, w.S)[:, inv]                           # [Hq, S]
    idx = torch.from_numpy(rows)
    got_out = np.stack([o[idx[h], h].double().numpy() for h in range(w.Hq)])
    got_lse = np.stack([l_[h, idx[h]].double().numpy() for h in range(w.Hq)])
    compare(got_out, got_lse, ref_out, ref_lse, TOL_BF16, "usp 128k gqa")


def test_all_to_all_128k_q_sampled_bitexact():
    """The q all-to-all of the 128k GQA workload in the launch configuration
    bench.py times (P = 8, 64 heads of 256-byte rows, 2 GiB; the tiled form
    with 4 positions x 64 heads per workgroup). The forward result is
    compared bit for bit with the oracle's on 4096 seeded destination rows
    plus the first and last row of every (rank, head) plane; the inverse
    restores every byte."""
    P, B, S, H, D = 8, 1, 131072, 64, 128
    Sp, Hp = S // P, H // P
    x = workloads.make_random((P, B, Sp, H, D), 990, torch.bfloat16)
    xd = x.to(DEV)
    y = torch.empty((P, B, Hp, S, D), dtype=torch.bfloat16, device=DEV)
    ra.ra_ulysses_all_to_all(xd, y, P)
    back = torch.empty_like(xd)
    ra.ra_ulysses_all_to_all(y, back, P, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back, xd)
    del back, xd
    ref = oracle.ulysses_all_to_all(x.view(torch.int16).numpy(), P)    # [P, B, S, H/P, D]
    rng = np.random.default_rng(990)
    j = rng.integers(0, P, 4096)
    hh = rng.integers(0, Hp, 4096)
    s = rng.integers(0, S, 4096)
    jj, hb = np.meshgrid(np.arange(P), np.arange(Hp), indexing="ij")
    j = np.concatenate([j, jj.ravel(), jj.ravel()])
    hh = np.concatenate([hh, hb.ravel(), hb.ravel()])
    s = np.concatenate([s, np.zeros(P * Hp, np.int64), np.full(P * Hp, S - 1)])
    got = y.view(torch.int16)[torch.from_numpy(j), 0, torch.from_numpy(hh),
                              torch.from_numpy(s)].cpu().numpy()
    print(f"  128k q all-to-all: {len(j)} rows compared", flush=True)
    np.testing.assert_array_equal(got, ref[j, 0, s, hh])
