"""Pins for the fp64 backward oracle (CPU only), independent of its own code.

  library  -- equals torch autograd through float64 scaled_dot_product_attention
  fd       -- equals central finite differences of sum(out * dout) (no torch)
  closed   -- single key / equal keys: dq = dk = 0, dv = sum of dout
  exact    -- the fp64 ring backward equals the full backward (the gradients
              are those of single-device attention), every layout
  invariant-- sum_j dv_j = sum_i dout_i and sum_j dk_j = 0 per KV head
  mutation -- planted mistakes in a copy of the oracle are caught
  count    -- backward_flops is twice the multiply-adds of a brute-force loop
              backward whose gradients equal the oracle's
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.fp64_bwd as good_bwd


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _autograd(q, k, v, dout, causal, mask=None):
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    g = q.shape[1] // k.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, 1), tv.repeat_interleave(g, 1),
        attn_mask=None if mask is None else torch.from_numpy(mask),
        is_causal=causal and mask is None)
    (o * torch.from_numpy(dout)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# ----------------------------------------------------------------- library
@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (1, 2, 2, 40, 16, True), (1, 4, 2, 33, 8, True), (2, 2, 1, 20, 32, False),
    (1, 8, 1, 17, 64, True),
])
def test_library_autograd(B, Hq, Hkv, S, D, causal):
    q, k, v = _rand((B, Hq, S, D), 1), _rand((B, Hkv, S, D), 2), _rand((B, Hkv, S, D), 3)
    dout = _rand((B, Hq, S, D), 4)
    got = oracle.attention_backward(q, k, v, dout, causal=causal)
    ref = _autograd(q, k, v, dout, causal)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_library_autograd_global_positions():
    """Causal rule on global positions (two key segments, queries in between)."""
    q, k, v = _rand((1, 2, 12, 8), 5), _rand((1, 2, 10, 8), 6), _rand((1, 2, 10, 8), 7)
    dout = _rand((1, 2, 12, 8), 8)
    qp = np.arange(20, 32)
    kp = np.concatenate([np.arange(0, 5), np.arange(25, 30)])
    mask = kp[None, :] <= qp[:, None]
    got = oracle.attention_backward(q, k, v, dout, causal=True, q_pos=qp, k_pos=kp)
    ref = _autograd(q, k, v, dout, False, mask=mask)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-12)


# ---------------------------------------------------------------------- fd
def test_finite_differences():
    q, k, v = _rand((1, 1, 5, 3), 9), _rand((1, 1, 5, 3), 10), _rand((1, 1, 5, 3), 11)
    dout = _rand((1, 1, 5, 3), 12)

    def loss(q_, k_, v_):
        return float((oracle.attention(q_, k_, v_, causal=True)[0] * dout).sum())

    grads = oracle.attention_backward(q, k, v, dout, causal=True)
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grads[which], num, atol=1e-8)


# ------------------------------------------------------------------ closed
def test_closed_equal_keys_and_single_key():
    """With all keys equal the scores of a row are equal, so ds sums to zero
    against a constant key: dq = 0, dk = 0, and dv_j = sum_i p_ij dout_i."""
    S, D = 7, 4
    q, dout = _rand((1, 1, S, D), 13), _rand((1, 1, S, D), 14)
    k = np.tile(_rand((1, 1, 1, D), 15), (1, 1, S, 1))
    v = _rand((1, 1, S, D), 16)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=True)
    np.testing.assert_allclose(dq, 0, atol=1e-13)
    np.testing.assert_allclose(dk.sum(axis=2), 0, atol=1e-12)
    # causal, uniform p: p_ij = 1/(i+1) for j <= i
    expect = np.array([sum(dout[0, 0, i] / (i + 1) for i in range(j, S)) for j in range(S)])
    np.testing.assert_allclose(dv[0, 0], expect, atol=1e-13)
    dq1, dk1, dv1 = oracle.attention_backward(q[:, :, :1], k[:, :, :1], v[:, :, :1],
                                              dout[:, :, :1], causal=True)
    np.testing.assert_allclose(dq1, 0, atol=1e-14)   # dp and delta sum in different orders
    np.testing.assert_allclose(dk1, 0, atol=1e-14)
    np.testing.assert_array_equal(dv1, dout[:, :, :1])


# ------------------------------------------------------------------- exact
@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("N,S,causal,Hq,Hkv", [(4, 32, True, 2, 1), (2, 24, False, 2, 2),
                                                (4, 48, True, 4, 2)])
def test_exact_ring_backward_equals_full(layout, N, S, causal, Hq, Hkv):
    D = 8
    q, k, v = _rand((1, Hq, S, D), 17), _rand((1, Hkv, S, D), 18), _rand((1, Hkv, S, D), 19)
    dout = _rand((1, Hq, S, D), 20)
    out, lse = oracle.attention(q, k, v, causal=causal)
    ref = oracle.attention_backward(q, k, v, dout, causal=causal)
    got = oracle.ring_attention_backward(q, k, v, dout, out, lse, N=N, layout=layout,
                                         causal=causal)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-12)


# --------------------------------------------------------------- invariant
def test_invariants_sum_dv_and_dk():
    B, Hq, Hkv, S, D = 1, 4, 2, 40, 8
    q, k, v = _rand((B, Hq, S, D), 21), _rand((B, Hkv, S, D), 22), _rand((B, Hkv, S, D), 23)
    dout = _rand((B, Hq, S, D), 24)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=True)
    for g in range(Hkv):
        heads = [h for h in range(Hq) if h // (Hq // Hkv) == g]
        np.testing.assert_allclose(dv[0, g].sum(0), sum(dout[0, h].sum(0) for h in heads),
                                   atol=1e-12)
        np.testing.assert_allclose(dk[0, g].sum(0), 0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_dq_rows_equal_full_backward(causal):
    q, k, v = _rand((1, 4, 30, 8), 29), _rand((1, 2, 30, 8), 30), _rand((1, 2, 30, 8), 31)
    dout = _rand((1, 4, 30, 8), 32)
    full = oracle.attention_backward(q, k, v, dout, causal=causal)[0]
    rows = np.array([[0, 7, 29], [3, 4, 5], [29, 28, 0], [10, 20, 1]])
    got = oracle.attention_backward_dq_rows(q, k, v, dout, rows, causal=causal)
    for h in range(4):
        np.testing.assert_allclose(got[0, h], full[0, h, rows[h]], atol=1e-12)


def _loop_backward_counting(q, k, v, dout, causal):
    """Brute-force backward of one head pair with plain loops over (i, j, d),
    counting the multiply-adds of its five products: the score recomputed,
    dP, and the dV, dK, dQ updates (the probabilities come from a first
    loop pass; delta from the forward output, as the pages' backward keeps
    it). Returns (dq, dk, dv, multiply-adds, allowed pairs)."""
    S, D = q.shape
    scale = 1.0 / math.sqrt(D)
    macs = 0
    ok = [[(not causal) or j <= i for j in range(S)] for i in range(S)]
    s = np.full((S, S), -np.inf)
    for i in range(S):
        for j in range(S):
            if ok[i][j]:
                acc = 0.0
                for d in range(D):
                    acc += q[i, d] * k[j, d]
                    macs += 1
                s[i, j] = scale * acc
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    out = p @ v                      # the forward's output (not a backward product)
    delta = (dout * out).sum(axis=1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    pairs = 0
    for i in range(S):
        for j in range(S):
            if not ok[i][j]:
                continue
            pairs += 1
            dp = 0.0
            for d in range(D):
                dp += dout[i, d] * v[j, d]
                macs += 1
            ds = p[i, j] * (dp - delta[i])
            for d in range(D):
                dv[j, d] += p[i, j] * dout[i, d]
                dk[j, d] += scale * ds * q[i, d]
                dq[i, d] += scale * ds * k[j, d]
                macs += 3
    return dq, dk, dv, macs, pairs


@pytest.mark.parametrize("causal", [True, False])
def test_backward_flops_counts_ten_d_per_pair(causal):
    """The useful-work count equals twice the multiply-adds a brute-force
    loop backward performs (whose gradients equal the oracle's)."""
    q, k, v, dout = (_rand((6, 4), 60 + i) for i in range(4))
    dq, dk, dv, macs, pairs = _loop_backward_counting(q, k, v, dout, causal)
    ref = oracle.attention_backward(q[None, None], k[None, None], v[None, None],
                                    dout[None, None], causal=causal)
    for a, b in zip((dq, dk, dv), ref):
        np.testing.assert_allclose(a, b[0, 0], atol=1e-12)
    assert pairs == (21 if causal else 36)
    assert oracle.backward_flops(1, 1, 4, pairs) == 2 * macs


# ---------------------------------------------------------------- mutation
def _mutant(old, new):
    with open(good_bwd.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_bwd_mutant")
    mod.__dict__["__package__"] = "oracle"
    mod.__dict__["__name__"] = "oracle.fp64_bwd_mutant"
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    return mod


def _battery(m):
    q, k, v = _rand((1, 2, 16, 8), 25), _rand((1, 1, 16, 8), 26), _rand((1, 1, 16, 8), 27)
    dout = _rand((1, 2, 16, 8), 28)
    ref = _autograd(q, k, v, dout, True)
    for a, b in zip(m.attention_backward(q, k, v, dout, causal=True), ref):
        np.testing.assert_allclose(a, b, atol=1e-10)
    out, lse = oracle.attention(q, k, v, causal=True)
    for layout in ("zigzag", "striped"):
        got = m.ring_attention_backward(q, k, v, dout, out, lse, N=4, layout=layout, causal=True)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, atol=1e-10)


MUTATIONS = {
    "drops_delta": ("ds = p * (dp - delta[:, None])\n            dq[b, h]",
                    "ds = p * dp\n            dq[b, h]"),
    "dk_no_scale": ("dk[b, g] += scale * (ds.T @ q[b, h])", "dk[b, g] += (ds.T @ q[b, h])"),
    "dv_uses_ds": ("dv[b, g] += p.T @ dout[b, h]", "dv[b, g] += ds.T @ dout[b, h]"),
    "dq_uses_v": ("dq[b, h] = scale * (ds @ k[b, g])", "dq[b, h] = scale * (ds @ v[b, g])"),
    "ring_block_no_delta": ("ds = p * (dp - delta[:, None])\n    return",
                            "ds = p * dp\n    return"),
    "ring_local_positions": ("q_pos=q_rows, k_pos=k_rows)",
                             "q_pos=np.arange(C), k_pos=np.arange(C))"),
    "ring_dk_to_home": ("dk[b, g, k_rows] += dk_b", "dk[b, g, q_rows] += dk_b"),
}


def test_unmutated_backward_passes_battery():
    _battery(good_bwd)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_planted_mistake_is_caught(name):
    m = _mutant(*MUTATIONS[name])
    with pytest.raises(AssertionError):
        _battery(m)
