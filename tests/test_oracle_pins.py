"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code (CPU only).

Each test names the pin it implements:
  library  -- the oracle equals torch's scaled_dot_product_attention / logsumexp
  hand     -- a hand-derived worked example (tests/golden)
  closed   -- closed forms (equal keys, zero queries, single key)
  exact    -- the fp64 ring equals full attention (the pages' exactness claim)
  causal   -- perturbing keys after position i leaves row i unchanged
  layout   -- zigzag / contiguous / striped assignment, with the pages' examples
  work     -- masked-in work per rank: brute force vs closed form
  merge    -- merge algebra against attention over the union of key sets
  schedule -- the 4-GPU ring figure
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, causal, scale, mask=None):
    """torch reference: float64 SDPA per head, GQA by repeating KV heads."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    group = tq.shape[1] // tk.shape[1]
    tk = tk.repeat_interleave(group, dim=1)
    tv = tv.repeat_interleave(group, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, is_causal=causal and mask is None, scale=scale)
    s = (tq @ tk.transpose(-1, -2)) * scale
    if mask is not None:
        s = s.masked_fill(~mask, -math.inf)
    elif causal:
        Sq, Sk = s.shape[-2:]
        s = s.masked_fill(torch.ones(Sq, Sk, dtype=torch.bool).triu(1), -math.inf)
    return out.numpy(), torch.logsumexp(s, dim=-1).numpy()


# ----------------------------------------------------------------- library
@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (1, 2, 2, 64, 16, True), (1, 2, 2, 64, 16, False),
    (2, 4, 2, 48, 8, True), (1, 6, 1, 33, 32, True), (1, 3, 3, 17, 64, False),
])
def test_library_sdpa(B, Hq, Hkv, S, D, causal):
    q = _rand((B, Hq, S, D), 1)
    k = _rand((B, Hkv, S, D), 2)
    v = _rand((B, Hkv, S, D), 3)
    scale = 1.0 / math.sqrt(D)
    out, lse = oracle.attention(q, k, v, causal=causal)
    ref_out, ref_lse = _sdpa(q, k, v, causal, scale)
    np.testing.assert_allclose(out, ref_out, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12, rtol=0)


def test_library_sdpa_global_positions():
    """Blocks with arbitrary global positions: the causal rule uses them."""
    rng = np.random.default_rng(7)
    Sq, Sk, D = 40, 56, 16
    q_pos = np.sort(rng.choice(200, Sq, replace=False))
    k_pos = np.sort(rng.choice(200, Sk, replace=False))
    q, k, v = _rand((1, 2, Sq, D), 4), _rand((1, 2, Sk, D), 5), _rand((1, 2, Sk, D), 6)
    out, lse = oracle.attention(q, k, v, causal=True, q_pos=q_pos, k_pos=k_pos)
    mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None])
    has_key = mask.any(dim=1).numpy()
    ref_out, ref_lse = _sdpa(q, k, v, False, 1 / math.sqrt(D), mask=mask)
    np.testing.assert_allclose(out[..., has_key, :], ref_out[..., has_key, :], atol=1e-12)
    np.testing.assert_allclose(lse[..., has_key], ref_lse[..., has_key], atol=1e-12)
    # rows with no allowed key: lse = -inf, out = 0
    assert np.all(lse[..., ~has_key] == -np.inf)
    assert np.all(out[..., ~has_key, :] == 0)


def test_library_row_sampling_matches_full():
    q, k, v = _rand((1, 3, 50, 8), 8), _rand((1, 3, 50, 8), 9), _rand((1, 3, 50, 8), 10)
    full_out, full_lse = oracle.attention(q, k, v, causal=True)
    rows = np.array([[0, 7, 49], [3, 4, 5], [49, 48, 1]])
    out, lse = oracle.attention(q, k, v, causal=True, rows=rows)
    for h in range(3):
        np.testing.assert_array_equal(out[0, h], full_out[0, h, rows[h]])
        np.testing.assert_array_equal(lse[0, h], full_lse[0, h, rows[h]])


# -------------------------------------------------------------------- hand
def test_hand_case_causal_s3():
    fx = _load("hand_case_causal_s3.json")
    q, k, v = (np.array(fx[n])[None, None] for n in ("q", "k", "v"))
    out, lse = oracle.attention(q, k, v, causal=fx["causal"], scale=fx["scale"])
    np.testing.assert_allclose(out[0, 0], np.array(fx["out"]), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.array(fx["lse"]), atol=1e-14)


def test_hand_case_embedded_d64():
    """The same case inside D=64 with the default scale 1/8: q[:,0]=8, rest 0."""
    fx = _load("hand_case_causal_s3.json")
    q = np.zeros((1, 1, 3, 64)); q[..., 0] = 8.0
    k = np.zeros((1, 1, 3, 64)); k[0, 0, :, 0] = np.array(fx["k"])[:, 0]
    v = np.zeros((1, 1, 3, 64)); v[0, 0, :, 0] = np.array(fx["v"])[:, 0]
    out, lse = oracle.attention(q, k, v, causal=True)
    np.testing.assert_allclose(out[0, 0, :, 0], np.array(fx["out"])[:, 0], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.array(fx["lse"]), atol=1e-14)
    assert np.all(out[0, 0, :, 1:] == 0)


# ------------------------------------------------------------------ closed
def test_closed_single_key():
    q, k, v = _rand((1, 1, 1, 8), 11), _rand((1, 1, 1, 8), 12), _rand((1, 1, 1, 8), 13)
    out, lse = oracle.attention(q, k, v, causal=True, scale=0.5)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 0.5 * q[0, 0, 0] @ k[0, 0, 0], atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_closed_equal_keys(causal):
    """All keys equal: weights are uniform over the allowed keys."""
    S, D = 37, 16
    q = _rand((1, 1, S, D), 14)
    krow = _rand((D,), 15)
    k = np.broadcast_to(krow, (1, 1, S, D)).copy()
    v = _rand((1, 1, S, D), 16)
    scale = 1 / math.sqrt(D)
    out, lse = oracle.attention(q, k, v, causal=causal)
    qk = scale * (q[0, 0] @ krow)
    if causal:
        n = np.arange(1, S + 1)
        exp_out = np.cumsum(v[0, 0], axis=0) / n[:, None]
        exp_lse = qk + np.log(n)
    else:
        exp_out = np.broadcast_to(v[0, 0].mean(axis=0), (S, D))
        exp_lse = qk + np.log(S)
    np.testing.assert_allclose(out[0, 0], exp_out, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], exp_lse, atol=1e-12)


def test_closed_zero_queries():
    S, D = 29, 8
    q = np.zeros((1, 1, S, D))
    k, v = _rand((1, 1, S, D), 17), _rand((1, 1, S, D), 18)
    out, lse = oracle.attention(q, k, v, causal=True)
    n = np.arange(1, S + 1)
    np.testing.assert_allclose(out[0, 0], np.cumsum(v[0, 0], 0) / n[:, None], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.log(n), atol=1e-12)


def test_closed_scale_shift():
    """A large score offset shared by every key cancels in out and shifts lse."""
    S, D = 20, 4
    q = np.zeros((1, 1, S, D)); q[..., 0] = 1.0
    k = _rand((1, 1, S, D), 19); k[..., 0] = 700.0   # exp(700*scale) alone would overflow fp64 sums
    v = _rand((1, 1, S, D), 20)
    out, lse = oracle.attention(q, k, v, causal=True, scale=1.0)
    k0 = k.copy(); k0[..., 0] = 0.0
    out0, lse0 = oracle.attention(q, k0, v, causal=True, scale=1.0)
    np.testing.assert_allclose(out, out0, atol=1e-12)
    np.testing.assert_allclose(lse, lse0 + 700.0, atol=1e-9)


# ------------------------------------------------------------------- exact
@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("N,S,causal,Hq,Hkv", [
    (4, 64, True, 2, 2), (4, 64, False, 2, 2), (2, 24, True, 4, 1),
    (8, 128, True, 4, 2), (1, 16, True, 1, 1), (3, 36, True, 3, 3),
])
def test_exact_ring_equals_full(layout, N, S, causal, Hq, Hkv):
    D = 8
    q, k, v = _rand((1, Hq, S, D), 21), _rand((1, Hkv, S, D), 22), _rand((1, Hkv, S, D), 23)
    ref_out, ref_lse = oracle.attention(q, k, v, causal=causal)
    out, lse = oracle.ring_attention(q, k, v, N=N, layout=layout, causal=causal)
    np.testing.assert_allclose(out, ref_out, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_exact_printed_O_new_needs_unnormalised_block():
    """Reading of the online-softmax O_new equation: with a NORMALISED block
    output in the printed formula the ring no longer equals full attention."""
    from oracle import fp64 as A
    rng = np.random.default_rng(24)
    D, C = 8, 16
    q, k1, v1, k2, v2 = (rng.standard_normal((C, D)) for _ in range(5))
    full_out, _ = oracle.attention(q[None, None], np.concatenate([k1, k2])[None, None],
                                   np.concatenate([v1, v2])[None, None], causal=False)
    m, l, O = np.full(C, -np.inf), np.zeros(C), np.zeros((C, D))
    for kk, vv in ((k1, v1), (k2, v2)):
        s = q @ kk.T / math.sqrt(D)
        mb = s.max(1); p = np.exp(s - mb[:, None]); lb = p.sum(1)
        m, l, O = A._online_softmax_update(m, l, O, mb, lb, (p @ vv) / lb[:, None])
    assert np.abs(O - full_out[0, 0]).max() > 1e-2


# ------------------------------------------------------------------ causal
def test_causal_future_keys_do_not_matter():
    S, D = 48, 8
    q, k, v = _rand((1, 2, S, D), 25), _rand((1, 2, S, D), 26), _rand((1, 2, S, D), 27)
    out, lse = oracle.attention(q, k, v, causal=True)
    for i in (0, 5, 31, 47):
        k2, v2 = k.copy(), v.copy()
        k2[..., i + 1:, :] = _rand(k2[..., i + 1:, :].shape, 28 + i)
        v2[..., i + 1:, :] = _rand(v2[..., i + 1:, :].shape, 90 + i)
        out2, lse2 = oracle.attention(q, k2, v2, causal=True)
        np.testing.assert_array_equal(out2[..., :i + 1, :], out[..., :i + 1, :])
        np.testing.assert_array_equal(lse2[..., :i + 1], lse[..., :i + 1])
        if i < S - 1:
            assert np.abs(out2[..., i + 1:, :] - out[..., i + 1:, :]).max() > 1e-3


def test_causal_local_offsets_negative_control():
    """Masking each rank's block with LOCAL offsets (causal per device, not
    globally) must not reproduce full attention."""
    S, N, D = 64, 4, 8
    C = S // N
    q, k, v = _rand((1, 1, S, D), 29), _rand((1, 1, S, D), 30), _rand((1, 1, S, D), 31)
    ref_out, _ = oracle.attention(q, k, v, causal=True)
    bad = np.zeros_like(ref_out)
    for r in range(N):
        rows = np.arange(r * C, (r + 1) * C)
        outs = []
        for src in range(N):
            cols = np.arange(src * C, (src + 1) * C)
            o, l_ = oracle.attention(q[..., rows, :], k[..., cols, :], v[..., cols, :], causal=True,
                                     q_pos=np.arange(C), k_pos=np.arange(C))
            outs.append((o, l_))
        o, l_ = outs[0]
        for o2, l2 in outs[1:]:
            o, l_ = oracle.merge(o, l_, o2, l2)
        bad[..., rows, :] = o
    assert np.abs(bad - ref_out).max() > 1e-2


# ------------------------------------------------------------------ layout
def test_layout_examples_from_page():
    fx = _load("layouts.json")
    for N, S, key in ((2, 8, "zigzag_S8_N2_rank_positions"), (4, 16, "zigzag_S16_N4_rank_positions")):
        for r, expected in enumerate(fx[key]):
            assert list(oracle.rank_positions(S, N, "zigzag", r)) == expected
    for r, expected in enumerate(fx["striped_S16_N4_rank_positions"]):
        assert list(oracle.rank_positions(16, 4, "striped", r)) == expected
    first, last = fx["contiguous_S8192_N8_rank0_first_last"]
    p = oracle.rank_positions(8192, 8, "contiguous", 0)
    assert p[0] == first and p[-1] == last and len(p) == 1024


@pytest.mark.parametrize("S,N", [(64, 4), (96, 3), (2048, 8), (32, 16)])
def test_layout_zigzag_properties(S, N):
    order = oracle.zigzag_order(S, N)
    assert sorted(order.tolist()) == list(range(S))           # a permutation
    c, C = S // (2 * N), S // N
    for r in range(N):
        pos = order[r * C:(r + 1) * C]
        chunks = sorted(set((pos // c).tolist()))
        assert len(chunks) == 2                                # two whole chunks
        assert chunks[0] < N <= chunks[1]                      # one early, one late
        for ch in chunks:
            assert sorted(pos[pos // c == ch].tolist()) == list(range(ch * c, (ch + 1) * c))
        assert pos[0] // c == chunks[0]                        # early chunk first
    x = _rand((2, S, 3), 32)
    assert np.array_equal(oracle.unpermute_rows(oracle.permute_rows(x, order, 1), order, 1), x)


@pytest.mark.parametrize("S,N", [(64, 4), (96, 3), (40, 8), (32, 32), (12, 1)])
def test_layout_striped_properties(S, N):
    """Brute force from the page's rule: token t lives on rank t mod N."""
    order = oracle.striped_order(S, N)
    assert sorted(order.tolist()) == list(range(S))
    C = S // N
    for r in range(N):
        pos = order[r * C:(r + 1) * C]
        assert pos.tolist() == [t for t in range(S) if t % N == r]
    x = _rand((2, S, 3), 35)
    assert np.array_equal(oracle.unpermute_rows(oracle.permute_rows(x, order, 1), order, 1), x)


# -------------------------------------------------------------------- work
@pytest.mark.parametrize("S,N", [(64, 4), (128, 8), (48, 2), (96, 3)])
def test_work_per_rank_closed_forms(S, N):
    c, C = S // (2 * N), S // N
    zz = oracle.pairs_per_rank_step(S, N, "zigzag", True)
    assert list(zz.sum(1)) == [(2 * N - 1) * c * c + c * (c + 1)] * N   # equal across ranks
    assert list(zz[:, 0]) == [2 * c * c + c] * N
    assert np.all(zz[:, 1:] == 2 * c * c)
    co = oracle.pairs_per_rank_step(S, N, "contiguous", True)
    assert list(co.sum(1)) == [r * C * C + C * (C + 1) // 2 for r in range(N)]
    assert zz.sum() == co.sum() == S * (S + 1) // 2
    nc = oracle.pairs_per_rank_step(S, N, "zigzag", False)
    assert np.all(nc == C * C)


@pytest.mark.parametrize("S,N", [(64, 4), (128, 8), (48, 2), (96, 3)])
def test_work_striped_closed_forms(S, N):
    """Striped: rank r against source s holds C(C+1)/2 allowed pairs per head if
    s <= r, else C(C-1)/2; rank r's total is C(r+1) + N C(C-1)/2."""
    C = S // N
    st = oracle.pairs_per_rank_step(S, N, "striped", True)
    for r in range(N):
        for k in range(N):
            s_ = oracle.ring_source(r, k, N)
            assert st[r, k] == (C * (C + 1) // 2 if s_ <= r else C * (C - 1) // 2)
    assert list(st.sum(1)) == [C * (r + 1) + N * C * (C - 1) // 2 for r in range(N)]
    assert st.sum() == S * (S + 1) // 2


def test_work_counts_s64_n4():
    assert list(oracle.pairs_per_rank_step(64, 4, "zigzag", True).sum(1)) == [520] * 4
    assert list(oracle.pairs_per_rank_step(64, 4, "contiguous", True).sum(1)) == [136, 392, 648, 904]


def test_score_term_grows_256x_from_8k_to_128k():
    """"Sequence and Context Parallelism", *The memory that data and tensor
    parallelism cannot touch*: a head's score matrix is S x S, so a 16x longer
    context (8k -> 128k) carries 256x the score term. The oracle's pair and
    flop counters reproduce the factor without a mask; with the causal mask
    the count is S(S+1)/2 (brute-forced at small S above), whose ratio tends
    to the same factor."""
    small, big = 8192, 131072
    p_small = oracle.useful_pairs(np.arange(small), np.arange(small), False)
    p_big = oracle.useful_pairs(np.arange(big), np.arange(big), False)
    assert p_big == 256 * p_small
    assert oracle.useful_flops(1, 64, 128, p_big) == 256 * oracle.useful_flops(1, 64, 128, p_small)
    causal_ratio = (big * (big + 1) // 2) / (small * (small + 1) // 2)
    assert abs(causal_ratio / 256 - 1) < 1e-3
    # the headline count: 4 D flops per allowed pair, 64 query heads, causal S = 2^17
    assert oracle.useful_flops(1, 64, 128, big * (big + 1) // 2) == 281477124194304


# ------------------------------------------------------------------- merge
def _partial(q, k, v, causal=False, q_pos=None, k_pos=None):
    return oracle.attention(q, k, v, causal=causal, q_pos=q_pos, k_pos=k_pos)


def test_merge_equals_union_and_algebra():
    D = 8
    q = _rand((1, 2, 10, D), 33)
    ks = [_rand((1, 2, n, D), 34 + n) for n in (5, 7, 3)]
    vs = [_rand((1, 2, n, D), 44 + n) for n in (5, 7, 3)]
    A, Bp, Cp = (_partial(q, k, v) for k, v in zip(ks, vs))
    union = _partial(q, np.concatenate(ks, 2), np.concatenate(vs, 2))
    ab = oracle.merge(*A, *Bp)
    ab_ref = _partial(q, np.concatenate(ks[:2], 2), np.concatenate(vs[:2], 2))
    np.testing.assert_allclose(ab[0], ab_ref[0], atol=1e-13)
    np.testing.assert_allclose(ab[1], ab_ref[1], atol=1e-13)
    ba = oracle.merge(*Bp, *A)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-14)
    left = oracle.merge(*ab, *Cp)
    right = oracle.merge(*A, *oracle.merge(*Bp, *Cp))
    np.testing.assert_allclose(left[0], union[0], atol=1e-13)
    np.testing.assert_allclose(right[0], union[0], atol=1e-13)
    np.testing.assert_allclose(left[1], union[1], atol=1e-13)
    empty = (np.zeros_like(A[0]), np.full_like(A[1], -np.inf))
    for x in (oracle.merge(*A, *empty), oracle.merge(*empty, *A)):
        np.testing.assert_array_equal(x[0], A[0])
        np.testing.assert_array_equal(x[1], A[1])
    both = oracle.merge(*empty, *empty)
    assert np.all(both[1] == -np.inf) and np.all(both[0] == 0)


def test_merge_masked_rows():
    """A causal block where some rows have no allowed key is the identity there."""
    D = 4
    q, k1, v1 = _rand((1, 1, 6, D), 50), _rand((1, 1, 6, D), 51), _rand((1, 1, 6, D), 52)
    k2, v2 = _rand((1, 1, 6, D), 53), _rand((1, 1, 6, D), 54)
    qp = np.arange(10, 16)
    A = _partial(q, k1, v1, True, qp, np.arange(0, 6))
    Bp = _partial(q, k2, v2, True, qp, np.arange(12, 18))   # rows 10, 11 see no key
    assert np.all(Bp[1][..., :2] == -np.inf)
    m = oracle.merge(*A, *Bp)
    np.testing.assert_array_equal(m[0][..., :2, :], A[0][..., :2, :])
    ref = _partial(q, np.concatenate([k1, k2], 2), np.concatenate([v1, v2], 2), True, qp,
                   np.concatenate([np.arange(0, 6), np.arange(12, 18)]))
    np.testing.assert_allclose(m[0], ref[0], atol=1e-13)
    np.testing.assert_allclose(m[1], ref[1], atol=1e-13)


# ---------------------------------------------------------------- schedule
def test_schedule_matches_4gpu_figure():
    fx = _load("ring_schedule_4gpu.json")
    sched = oracle.ring_schedule(fx["N"])
    for r, (s0, s1) in enumerate(fx["source_by_rank_step01"]):
        assert sched[r, 0] == s0 and sched[r, 1] == s1
    # every rank sees every source exactly once
    for N in (1, 2, 5, 8, 16):
        s = oracle.ring_schedule(N)
        assert all(sorted(row) == list(range(N)) for row in s.tolist())
