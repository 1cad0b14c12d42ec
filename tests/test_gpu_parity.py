"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Tolerances: bf16 inputs (fp32 accumulation) out max-abs <= 2e-2, mean-abs <=
2e-3, lse max-abs <= 1e-3; fp32 inputs <= 1e-4; the zigzag permute and
the masked-row / empty-block identities are bit-exact. The striped layout
(token t on rank t mod N) is covered by its own permute, block and ring cases.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL_BF16, TOL_F32, check_rows, compare, pooled_attention

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_context_parallelism_flash_amd")
DEV = "cuda"


def _rnd(shape, seed, dtype, scale=1.0):
    return workloads.make_random(shape, seed, dtype, scale)


def _pos_array(desc, rows):
    """Positions of a (nseg, seg_len, start0[, start1[, stride]]) descriptor."""
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


# ---------------------------------------------------------------- permute
@pytest.mark.parametrize("shape,N,dtype,seq_dim", [
    ((2, 3, 64, 8), 4, torch.bfloat16, -2),
    ((1, 2, 1024), 8, torch.float32, -1),
    ((1, 5, 48, 3), 3, torch.int16, -2),      # 6-byte rows: 2-byte accesses
    ((1, 1, 4096, 128), 16, torch.bfloat16, -2),
])
def test_zigzag_permute_bitexact(shape, N, dtype, seq_dim):
    g = torch.Generator().manual_seed(5)
    src = torch.randint(-30000, 30000, shape, generator=g, dtype=torch.int32).to(dtype)
    S = shape[seq_dim]
    order = oracle.zigzag_order(S, N)
    expect = np.take(src.numpy() if dtype != torch.bfloat16 else src.view(torch.int16).numpy(),
                     order, axis=seq_dim % len(shape))
    s_dev = src.to(DEV)
    dst = torch.empty_like(s_dev)
    ra.ra_zigzag_permute(s_dev, dst, N, inverse=False, seq_dim=seq_dim)
    back = torch.empty_like(s_dev)
    ra.ra_zigzag_permute(dst, back, N, inverse=True, seq_dim=seq_dim)
    torch.cuda.synchronize()
    got = dst.cpu()
    got = got.view(torch.int16).numpy() if dtype == torch.bfloat16 else got.numpy()
    assert np.array_equal(got, expect)
    assert torch.equal(back.cpu().view(torch.int16) if dtype == torch.bfloat16 else back.cpu(),
                       src.view(torch.int16) if dtype == torch.bfloat16 else src)


@pytest.mark.parametrize("shape,N,dtype,seq_dim", [
    ((2, 3, 64, 8), 4, torch.bfloat16, -2),
    ((1, 2, 1024), 8, torch.float32, -1),
    ((1, 5, 48, 3), 3, torch.int16, -2),      # 6-byte rows: 2-byte accesses
    ((1, 1, 4096, 128), 16, torch.bfloat16, -2),
    ((1, 2, 96, 300), 3, torch.float32, -2),   # 1200-byte rows: longer than one block
])
def test_striped_permute_bitexact(shape, N, dtype, seq_dim):
    g = torch.Generator().manual_seed(6)
    src = torch.randint(-30000, 30000, shape, generator=g, dtype=torch.int32).to(dtype)
    S = shape[seq_dim]
    order = oracle.striped_order(S, N)
    as_np = (lambda t: t.view(torch.int16).numpy()) if dtype == torch.bfloat16 else (lambda t: t.numpy())
    expect = np.take(as_np(src), order, axis=seq_dim % len(shape))
    s_dev = src.to(DEV)
    dst = torch.empty_like(s_dev)
    ra.ra_striped_permute(s_dev, dst, N, inverse=False, seq_dim=seq_dim)
    back = torch.empty_like(s_dev)
    ra.ra_striped_permute(dst, back, N, inverse=True, seq_dim=seq_dim)
    torch.cuda.synchronize()
    assert np.array_equal(as_np(dst.cpu()), expect)
    assert np.array_equal(as_np(back.cpu()), as_np(src))


# ---------------------------------------------------------------- merge
@pytest.mark.parametrize("rows,D", [(1000, 128), (77, 5), (4096, 64)])
def test_lse_merge_vs_oracle(rows, D):
    g = torch.Generator().manual_seed(rows)
    out_a = torch.randn(rows, D, generator=g)
    out_b = torch.randn(rows, D, generator=g)
    lse_a = torch.randn(rows, generator=g) * 5
    lse_b = torch.randn(rows, generator=g) * 5
    lse_a[::7] = -math.inf       # empty running state
    lse_b[::5] = -math.inf       # empty partial
    out_a[::7] = 0
    out_b[::5] = 0
    ref_out, ref_lse = oracle.merge(out_a, lse_a, out_b, lse_b)
    o, l_ = out_a.to(DEV), lse_a.to(DEV)
    ra.ra_lse_merge(o, l_, out_b.to(DEV), lse_b.to(DEV))
    torch.cuda.synchronize()
    compare(_np(o), _np(l_), ref_out, ref_lse, dict(max_abs=1e-5, mean_abs=1e-6, lse=1e-5),
            f"merge rows={rows} D={D}")
    both = (lse_a == -math.inf) & (lse_b == -math.inf)
    assert torch.all(l_.cpu()[both] == -math.inf) and torch.all(o.cpu()[both] == 0)


def test_zigzag_permute_128k_q_sampled_bitexact():
    """The 2 GiB q permute of the 128k GQA workload in the launch configuration
    bench.py times (N = 8, 16 chunks of 8192 rows of 256 bytes per head
    plane): 4096 seeded destination rows plus every chunk's first and last row
    of every head, bit for bit against the oracle's zigzag order; the inverse
    restores every byte."""
    w = workloads.HEADLINE
    B, H, S, D, N = w.B, w.Hq, w.S, w.D, w.N
    src = workloads.make_random((B, H, S, D), 991, torch.bfloat16)
    s_dev = src.to(DEV)
    dst = torch.empty_like(s_dev)
    ra.ra_zigzag_permute(s_dev, dst, N)
    back = torch.empty_like(s_dev)
    ra.ra_zigzag_permute(dst, back, N, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back, s_dev)
    del back, s_dev
    order = oracle.zigzag_order(S, N)         # destination row t holds sequence row order[t]
    rng = np.random.default_rng(991)
    h = rng.integers(0, H, 4096)
    t = rng.integers(0, S, 4096)
    c = S // (2 * N)
    ends = np.concatenate([np.arange(2 * N) * c, np.arange(2 * N) * c + c - 1])
    hh, ee = np.meshgrid(np.arange(H), ends, indexing="ij")
    h = np.concatenate([h, hh.ravel()])
    t = np.concatenate([t, ee.ravel()])
    got = dst.view(torch.int16)[0, torch.from_numpy(h), torch.from_numpy(t)].cpu().numpy()
    want = src.view(torch.int16).numpy()[0, h, order[t]]
    print(f"  128k q zigzag permute: {len(t)} rows compared", flush=True)
    np.testing.assert_array_equal(got, want)


def test_lse_merge_rank_state_sampled():
    """ra_lse_merge on one rank's running state of the 128k GQA workload (64
    heads x 16384 rows of D = 128, the size bench.py times), with empty rows
    on either side: 4096 seeded rows plus the first and last against the
    oracle's merge of the same rows."""
    rows, D = 64 * 16384, 128
    g = torch.Generator().manual_seed(992)
    out_a = torch.randn(rows, D, generator=g)
    out_b = torch.randn(rows, D, generator=g)
    lse_a = torch.randn(rows, generator=g) * 5
    lse_b = torch.randn(rows, generator=g) * 5
    lse_a[::7] = -math.inf
    lse_b[::5] = -math.inf
    out_a[::7] = 0
    out_b[::5] = 0
    o, l_ = out_a.to(DEV), lse_a.to(DEV)
    ra.ra_lse_merge(o, l_, out_b.to(DEV), lse_b.to(DEV))
    torch.cuda.synchronize()
    pick = np.concatenate([np.random.default_rng(992).choice(rows, 4096, replace=False),
                           [0, rows - 1]])
    idx = torch.from_numpy(pick)
    ref_out, ref_lse = oracle.merge(out_a[idx], lse_a[idx], out_b[idx], lse_b[idx])
    compare(_np(o[idx.to(DEV)]), _np(l_[idx.to(DEV)]), ref_out, ref_lse,
            dict(max_abs=1e-5, mean_abs=1e-6, lse=1e-5), f"merge {rows} rows, {len(pick)} compared")


# ---------------------------------------------------------------- block
def _block_case(dtype, D, Cq, Ck, q_pos, k_pos, causal, Hq=4, Hkv=2, kv_map=None, seed=0,
                accumulate=False):
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = _rnd((1, Hq, Cq, D), seed + 1, dt)
    k = _rnd((1, Hkv, Ck, D), seed + 2, dt)
    v = _rnd((1, Hkv, Ck, D), seed + 3, dt)
    qp, kp = _pos_array(q_pos, Cq), _pos_array(k_pos, Ck)
    ref_out, ref_lse = oracle.attention(q, k, v, causal=causal, kv_head_of_q=kv_map,
                                        q_pos=qp, k_pos=kp)
    if accumulate:
        # a running state from an earlier block of keys at positions below kp
        k0 = _rnd((1, Hkv, 96, D), seed + 4, dt)
        v0 = _rnd((1, Hkv, 96, D), seed + 5, dt)
        o0, l0 = oracle.attention(q, k0, v0, causal=causal, kv_head_of_q=kv_map, q_pos=qp,
                                  k_pos=np.arange(96) + int(kp.min()) - 96 if len(kp) else
                                  np.arange(96))
        out = torch.from_numpy(o0).float()
        lse = torch.from_numpy(l0).float()
        ref_out, ref_lse = oracle.merge(out, lse, ref_out, ref_lse)
    else:
        out = torch.full((1, Hq, Cq, D), 7.0)      # garbage: must be overwritten
        lse = torch.full((1, Hq, Cq), 3.0)
    o, l_ = out.to(DEV), lse.to(DEV)
    ra.ra_block_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), o, l_, q_pos=q_pos, k_pos=k_pos,
                         kv_head_of_q=kv_map, causal=causal, accumulate=accumulate)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    compare(_np(o), _np(l_), ref_out, ref_lse, tol,
            f"block {dtype} D={D} Cq={Cq} Ck={Ck} qpos={q_pos} kpos={k_pos} acc={accumulate}")


BLOCK_CASES = [
    # Cq, Ck, q_pos, k_pos, causal
    (128, 64, None, None, True),                      # one diagonal tile
    (300, 200, None, None, True),                     # ragged q and k tiles
    (257, 513, (1, 257, 1000), None, True),           # all keys visible: no mask
    (256, 256, (2, 128, 0, 768), (2, 128, 256, 512), True),  # zigzag-like: empty + full
    (384, 320, (2, 192, 100, 700), (2, 160, 0, 600), True),  # diagonals inside both segments
    (200, 333, None, None, False),
    (1, 1, None, None, True),
    (5, 3, (1, 5, 2), None, True),
    # strided positions (the striped split): rank 1 against rank 2 of 4 is a
    # strictly lower triangle, rank 3 against rank 0 an inclusive one
    (256, 256, (1, 256, 1, 0, 4), (1, 256, 2, 0, 4), True),
    (300, 200, (1, 300, 3, 0, 4), (1, 200, 0, 0, 4), True),
    (256, 192, (2, 128, 0, 700, 3), (1, 192, 1, 0, 5), True),   # unequal strides
    (130, 70, (1, 130, 0, 0, 7), (1, 70, 5, 0, 7), False),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", range(len(BLOCK_CASES)))
def test_block_attn_vs_oracle(dtype, D, case):
    Cq, Ck, qp, kp, causal = BLOCK_CASES[case]
    _block_case(dtype, D, Cq, Ck, qp, kp, causal, seed=10 * case)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_attn_accumulate_and_gqa_map(dtype):
    _block_case(dtype, 128, 300, 200, (1, 300, 500), (1, 200, 400), True, Hq=4, Hkv=2,
                kv_map=[1, 0, 1, 0], seed=3, accumulate=True)
    _block_case(dtype, 64, 200, 264, None, None, False, Hq=6, Hkv=3, seed=4, accumulate=True)


def test_block_hand_case():
    """The hand-derived S=3 example embedded in D=64 (scale 1/8, q[:,0]=8)."""
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_case_causal_s3.json")) as f:
        fx = json.load(f)
    for dt, tol in ((torch.float32, 1e-6), (torch.bfloat16, 2e-2)):
        q = torch.zeros(1, 1, 3, 64)
        q[..., 0] = 8.0
        k = torch.zeros(1, 1, 3, 64)
        k[0, 0, :, 0] = torch.tensor(fx["k"])[:, 0]
        v = torch.zeros(1, 1, 3, 64)
        v[0, 0, :, 0] = torch.tensor(fx["v"])[:, 0]
        q, k, v = q.to(dt), k.to(dt), v.to(dt)
        o = torch.zeros(1, 1, 3, 64, device=DEV)
        l_ = torch.zeros(1, 1, 3, device=DEV)
        ra.ra_block_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), o, l_, causal=True)
        torch.cuda.synchronize()
        exp_out = np.array(fx["out"])[:, 0]
        exp_lse = np.array(fx["lse"])
        if dt == torch.bfloat16:   # the bf16-rounded keys move the exact answer slightly
            exp_out, exp_lse = (x[0, 0] for x in oracle.attention(q, k, v, causal=True))
            exp_out = exp_out[:, 0]
        assert np.abs(_np(o)[0, 0, :, 0] - exp_out).max() <= tol
        assert np.abs(_np(l_)[0, 0] - exp_lse).max() <= tol
        assert torch.all(o[0, 0, :, 1:] == 0)


def test_block_vt_rows_past_4gib_closed_form():
    """A bf16 key block so long that the transposed-V rows of one head start
    more than 4 GiB apart (D = 64, Ck = 2^25 + 2^20: row 63 begins at
    63 * Ck * 2 bytes > 2^32), so the tile loads take their 64-bit offset path.

    Keys and values are zero except three needle rows, each with score 30
    (q[:, 0] = 8, k[needle, 0] = 30, scale 1/8) and its values in its own
    third of the d columns. Closed form: every background score is 0, so with
    Z = 3 e^30 + (Ck - 3), out[d] = e^30 v_n[d] / Z and lse = ln Z (the
    background adds ~1e-6 relative, below the tolerance)."""
    D, Hq, Hkv, Cq = 64, 2, 1, 64
    Ck = (1 << 25) + (1 << 20)
    q = torch.zeros(1, Hq, Cq, D, dtype=torch.bfloat16, device=DEV)
    q[..., 0] = 8.0
    k = torch.zeros(1, Hkv, Ck, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    rows = (100, (1 << 24) + 12345, Ck - 7)   # early, middle, last tile
    cols = ((0, 21), (21, 42), (42, 64))
    expect_v = np.zeros(D)
    for n, (r, (c0, c1)) in enumerate(zip(rows, cols)):
        k[0, 0, r, 0] = 30.0
        vals = np.arange(c0, c1) * 0.25 - 4.0 + n   # exact in bf16
        v[0, 0, r, c0:c1] = torch.tensor(vals, dtype=torch.bfloat16)
        expect_v[c0:c1] = vals
    out = torch.zeros(1, Hq, Cq, D, device=DEV)
    lse = torch.zeros(1, Hq, Cq, device=DEV)
    ra.ra_block_attn_fwd(q, k, v, out, lse, causal=False)
    torch.cuda.synchronize()
    del k, v
    Z = 3.0 * math.exp(30.0) + (Ck - 3)
    exp_out = expect_v * math.exp(30.0) / Z
    o, l_ = _np(out), _np(lse)
    assert np.abs(o - exp_out).max() <= 1e-4
    assert np.abs(l_ - math.log(Z)).max() <= 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_future_keys_identity(dtype):
    """A block entirely after the queries: accumulate leaves the state bit-identical,
    overwrite gives out=0, lse=-inf. An empty key block behaves the same way."""
    q = _rnd((1, 2, 200, 128), 1, dtype).to(DEV)
    k = _rnd((1, 2, 130, 128), 2, dtype).to(DEV)
    v = _rnd((1, 2, 130, 128), 3, dtype).to(DEV)
    out0 = torch.randn(1, 2, 200, 128, device=DEV)
    lse0 = torch.randn(1, 2, 200, device=DEV)
    for kk, vv, kp in ((k, v, (1, 130, 500)), (k[:, :, :0], v[:, :, :0], None)):
        o, l_ = out0.clone(), lse0.clone()
        ra.ra_block_attn_fwd(q, kk, vv, o, l_, q_pos=(1, 200, 0), k_pos=kp, causal=True,
                             accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(o, out0) and torch.equal(l_, lse0)
        ra.ra_block_attn_fwd(q, kk, vv, o, l_, q_pos=(1, 200, 0), k_pos=kp, causal=True,
                             accumulate=False)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(l_ == -math.inf)


# ---------------------------------------------------------------- ring
def _ring_check(w, rows=None, tol=None, copy_stream=True):
    q, k, v = workloads.make_inputs(w)
    B, Hq, S, D = q.shape
    r = ra.RingRunner(B, Hq, w.Hkv, S, D, q.dtype, w.N, w.layout, w.causal, device=DEV,
                      copy_stream=copy_stream)
    out = torch.empty(q.shape, dtype=q.dtype, device=DEV)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    r(q.to(DEV), k.to(DEV), v.to(DEV), out, lse)
    torch.cuda.synchronize()
    tol = tol or (TOL_F32 if w.dtype == "f32" else TOL_BF16)
    if rows is None:
        ref_out, ref_lse = (pooled_attention(q, k, v, causal=w.causal,
                                             rows=np.tile(np.arange(S), (Hq, 1)))
                            if B == 1 and S >= 4096 else
                            oracle.attention(q, k, v, causal=w.causal))
        if B == 1 and S >= 4096:
            ref_out, ref_lse = ref_out[None], ref_lse[None]
        got_out, got_lse = _np(out), _np(lse)
    else:
        ref_out, ref_lse = pooled_attention(q, k, v, causal=w.causal, rows=rows)
        idx = torch.from_numpy(rows)
        o = out[0].cpu()
        got_out = np.stack([o[h, idx[h]].double().numpy() for h in range(Hq)])
        got_lse = np.stack([lse[0, h].cpu()[idx[h]].double().numpy() for h in range(Hq)])
    compare(got_out, got_lse, ref_out, ref_lse, tol, f"ring {w.name}")
    return out, lse


SMALL_RINGS = [
    workloads.Workload("ragged_zigzag_gqa", B=1, Hq=4, Hkv=2, D=128, S=1000, dtype="bf16",
                       seed=21, causal=True, N=4, layout="zigzag"),
    workloads.Workload("batch2_contig_d64", B=2, Hq=4, Hkv=1, D=64, S=768, dtype="bf16",
                       seed=22, causal=True, N=3, layout="contiguous"),
    workloads.Workload("single_rank", B=1, Hq=2, Hkv=2, D=128, S=640, dtype="bf16", seed=23,
                       causal=True, N=1, layout="zigzag"),
    workloads.Workload("f32_zigzag_ragged", B=1, Hq=2, Hkv=1, D=128, S=600, dtype="f32",
                       seed=24, causal=True, N=3, layout="zigzag"),
    workloads.Workload("stress_scores_q_x8", B=1, Hq=2, Hkv=2, D=128, S=2048, dtype="bf16",
                       seed=25, causal=True, N=4, layout="zigzag"),
    workloads.Workload("contig_s8192_n8_rank0_0_1023", B=1, Hq=2, Hkv=2, D=128, S=8192,
                       dtype="bf16", seed=26, causal=True, N=8, layout="contiguous"),
    workloads.Workload("striped_gqa", B=1, Hq=4, Hkv=2, D=128, S=1024, dtype="bf16", seed=27,
                       causal=True, N=4, layout="striped"),
    workloads.Workload("striped_ragged_n8", B=1, Hq=2, Hkv=1, D=128, S=1000, dtype="bf16",
                       seed=28, causal=True, N=8, layout="striped"),
    workloads.Workload("striped_f32_d64", B=2, Hq=2, Hkv=1, D=64, S=600, dtype="f32", seed=29,
                       causal=True, N=3, layout="striped"),
    # non-causal zigzag with two batches and two query heads per KV head
    workloads.Workload("noncausal_zigzag_b2_gqa2_d64", B=2, Hq=6, Hkv=3, D=64, S=1200,
                       dtype="bf16", seed=30, causal=False, N=3, layout="zigzag"),
    # five query heads per KV head, five ranks, 101-token chunks (ragged tiles)
    workloads.Workload("causal_zigzag_gqa5_n5_ragged", B=1, Hq=5, Hkv=1, D=64, S=1010,
                       dtype="bf16", seed=31, causal=True, N=5, layout="zigzag"),
]


@pytest.mark.parametrize("w", SMALL_RINGS, ids=[w.name for w in SMALL_RINGS])
def test_ring_small_vs_oracle(w):
    if w.name.startswith("stress"):
        # large scores exercise the running-max rescale: q scaled by 8
        q, k, v = workloads.make_inputs(w)
        q = (q.float() * 8).to(q.dtype)
        out, lse = ra.ring_attention_sim(q.to(DEV), k.to(DEV), v.to(DEV), N=w.N,
                                         layout=w.layout, causal=True)
        torch.cuda.synchronize()
        ref = oracle.attention(q, k, v, causal=True)
        compare(_np(out), _np(lse), *ref, TOL_BF16, w.name)
        return
    _ring_check(w)


@pytest.mark.parametrize("idx", [0, 1])
def test_ring_config_all_rows(idx):
    """The tiny fp32 ring and the non-causal 8k ring, every row checked."""
    _ring_check(workloads.WORKLOADS[idx])


def _rows_or_all(w, default_random, fixed=None):
    """Rows checked per head: every row when ``RA_ORACLE_ROWS`` (default
    ``default_random``; "all" or a number >= S) covers the sequence, else that
    many seeded rows per head plus every chunk's first and last row."""
    n = os.environ.get("RA_ORACLE_ROWS", str(default_random))
    n = w.S if n == "all" else int(n)
    if n >= w.S:
        rows = np.tile(np.arange(w.S), (w.Hq, 1))
    else:
        rows = check_rows(w.S, w.Hq, n, w.seed, 2 * w.N, fixed=fixed)
    print(f"  {w.name}: {rows.shape[1]} oracle rows per head x {w.Hq} heads "
          f"(S={w.S})", flush=True)
    return rows


def test_ring_config_causal_zigzag_32k_all_rows():
    """The 32k MHA zigzag ring on every row of every head."""
    w = workloads.WORKLOADS[2]
    _ring_check(w, rows=_rows_or_all(w, "all"))


def test_ring_headline_gqa_128k_sampled():
    """The 128k GQA zigzag ring: 4096 seeded rows per head plus every chunk's
    first and last row (so row S-1, which sees every key, on every head)."""
    w = workloads.HEADLINE
    rows = _rows_or_all(w, 4096)
    assert np.all(rows[:, -1] == w.S - 1) and np.all(rows[:, 0] == 0)
    _ring_check(w, rows=rows)


def test_ring_striped_gqa_128k_sampled():
    """Seeded rows plus each striped rank's first and last rows (positions
    0..N-1 and S-N..S-1) and the 2N chunk boundaries, the same count per head."""
    w = workloads.STRIPED_128K
    fixed = np.concatenate([np.arange(w.N), w.S - w.N + np.arange(w.N)])
    _ring_check(w, rows=_rows_or_all(w, 256, fixed=fixed))


def test_ring_million_token_mqa_sampled():
    """The 1M-token MQA zigzag ring: 4096 seeded rows per head plus every
    chunk's first and last row."""
    w = workloads.WORKLOADS[4]
    rows = _rows_or_all(w, 4096)
    assert np.all(rows[:, -1] == w.S - 1)
    _ring_check(w, rows=rows)


def test_ring_zigzag_equals_contiguous_and_no_copy_stream():
    base = dict(B=1, Hq=4, Hkv=2, D=128, S=4096, dtype="bf16", seed=31, causal=True, N=8)
    wz = workloads.Workload("z", layout="zigzag", **base)
    wc = workloads.Workload("c", layout="contiguous", **base)
    oz, lz = _ring_check(wz)
    oc, lc = _ring_check(wc)
    o1, l1 = _ring_check(wz, copy_stream=False)
    assert torch.equal(oz, o1) and torch.equal(lz, l1)
    assert (oz.float() - oc.float()).abs().max().item() <= 2e-2
    assert (lz - lc).abs().max().item() <= 1e-3


def test_ring_striped_equals_contiguous():
    base = dict(B=1, Hq=4, Hkv=2, D=128, S=4096, dtype="bf16", seed=32, causal=True, N=8)
    os_, ls_ = _ring_check(workloads.Workload("s", layout="striped", **base))
    oc, lc = _ring_check(workloads.Workload("c", layout="contiguous", **base))
    assert (os_.float() - oc.float()).abs().max().item() <= 2e-2
    assert (ls_ - lc).abs().max().item() <= 1e-3


def test_ring_causality_perturbation_bitexact():
    w = workloads.Workload("perturb", B=1, Hq=2, Hkv=1, D=128, S=2048, dtype="bf16", seed=41,
                           causal=True, N=4, layout="zigzag")
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    o1, l1 = ra.ring_attention_sim(q, k, v, N=w.N, layout=w.layout)
    i = 1000
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i + 1:] = _rnd(k2[:, :, i + 1:].shape, 99, torch.bfloat16).to(DEV)
    v2[:, :, i + 1:] = _rnd(v2[:, :, i + 1:].shape, 98, torch.bfloat16).to(DEV)
    o2, l2 = ra.ring_attention_sim(q, k2, v2, N=w.N, layout=w.layout)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :i + 1], o2[:, :, :i + 1])
    assert torch.equal(l1[:, :, :i + 1], l2[:, :, :i + 1])
    assert not torch.equal(o1[:, :, i + 1:], o2[:, :, i + 1:])


def test_ring_deterministic_under_copy_delay():
    """Delaying the copy stream before the call must not change a single bit:
    every compute step waits for its block to land."""
    w = workloads.Workload("delay", B=1, Hq=8, Hkv=2, D=128, S=8192, dtype="bf16", seed=51,
                           causal=True, N=8, layout="zigzag")
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    r = ra.RingRunner(1, 8, 2, w.S, 128, torch.bfloat16, w.N, "zigzag", True, device=DEV)
    out1 = torch.empty_like(q)
    lse1 = torch.empty(1, 8, w.S, device=DEV)
    r(q, k, v, out1, lse1)
    torch.cuda.synchronize()
    out2, lse2 = torch.empty_like(out1), torch.empty_like(lse1)
    qr, kr, vr = r.permute_inputs(q, k, v)
    with torch.cuda.stream(r.copy_stream):
        torch.cuda._sleep(50_000_000)
    r.ring(qr, kr, vr)
    r.unpermute_outputs(out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_ring_copy_ahead_of_compute_waits_for_freed_slot():
    """The write-after-read side of the double buffer. With 64 query heads on
    one KV head, a block copy moves 1 MiB while the attention step that reads
    the other slot does ~7e10 flops, so the copy stream is always ahead of the
    compute stream; the compute stream is also held back by a sleep before
    the ring. A copy into a slot may start only after the step that last read
    it has finished (its "freed" event); if it did not wait, later blocks
    would overwrite slots still being read. The result must be bit-identical
    to the same ring on a single stream, where no overlap exists."""
    w = workloads.Workload("war", B=1, Hq=64, Hkv=1, D=128, S=16384, dtype="bf16", seed=52,
                           causal=True, N=8, layout="zigzag")
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    one = ra.RingRunner(1, 64, 1, w.S, 128, torch.bfloat16, w.N, "zigzag", True, device=DEV,
                        copy_stream=False)
    two = ra.RingRunner(1, 64, 1, w.S, 128, torch.bfloat16, w.N, "zigzag", True, device=DEV)
    out1, lse1 = torch.empty_like(q), torch.empty(1, 64, w.S, device=DEV)
    one(q, k, v, out1, lse1)
    torch.cuda.synchronize()
    qr, kr, vr = two.permute_inputs(q, k, v)
    for _ in range(2):
        torch.cuda._sleep(50_000_000)          # the compute (current) stream waits
        two.ring(qr, kr, vr)
        out2, lse2 = torch.empty_like(out1), torch.empty_like(lse1)
        two.unpermute_outputs(out2, lse2)
        torch.cuda.synchronize()
        assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


RACE_RINGS = [
    workloads.Workload("race_a_zigzag", B=1, Hq=8, Hkv=2, D=128, S=8192, dtype="bf16", seed=61,
                       causal=True, N=8, layout="zigzag"),
    workloads.Workload("race_b_contig", B=1, Hq=4, Hkv=4, D=64, S=4096, dtype="bf16", seed=62,
                       causal=True, N=4, layout="contiguous"),
]


def test_ring_concurrent_host_threads_bitexact():
    """Two host threads enqueue rings at the same time, each on its own compute
    and copy streams with its own workspace (the binding's library calls
    release the interpreter lock, so the two enqueue loops interleave in the
    library). Every call creates its own ring events, so a wait cannot bind
    to the other thread's record: each result is bit-identical to the same
    ring run alone."""
    import threading
    runners, inputs, ref = [], [], []
    for w in RACE_RINGS:
        r = ra.RingRunner(w.B, w.Hq, w.Hkv, w.S, w.D, torch.bfloat16, w.N, w.layout, w.causal,
                          device=DEV)
        q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
        out, lse = torch.empty_like(q), torch.empty(w.B, w.Hq, w.S, device=DEV)
        r(q, k, v, out, lse)
        torch.cuda.synchronize()
        runners.append(r)
        inputs.append((q, k, v))
        ref.append((out, lse))
    results = [[], []]
    errors = []
    start = threading.Barrier(2)

    def work(i):
        try:
            s = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(s):
                outs = [(torch.empty_like(ref[i][0]), torch.empty_like(ref[i][1]))
                        for _ in range(4)]
                start.wait()
                for out, lse in outs:
                    runners[i](*inputs[i], out, lse)
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a ring thread did not finish"
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == 4
        for out, lse in results[i]:
            assert torch.equal(out, ref[i][0]) and torch.equal(lse, ref[i][1]), RACE_RINGS[i].name


def test_ring_repeat_bitexact_noncausal_8k():
    """Repeated runs are bit-identical. This workload (32 key tiles per
    launch) exposed a missing wait on the direct global->LDS tile loads
    before the key-loop barrier: results then varied from run to run."""
    w = workloads.WORKLOADS[1]
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    r = ra.RingRunner(w.B, w.Hq, w.Hkv, w.S, w.D, q.dtype, w.N, w.layout, w.causal, device=DEV)
    outs = []
    for _ in range(3):
        out = torch.empty_like(q)
        lse = torch.empty(w.B, w.Hq, w.S, device=DEV)
        r(q, k, v, out, lse)
        torch.cuda.synchronize()
        outs.append((out, lse))
    for out, lse in outs[1:]:
        assert torch.equal(out, outs[0][0]) and torch.equal(lse, outs[0][1])
