"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies the oracle's source text, plants one plausible mistake (a
dropped term, a wrong sign, a wrong index, a swapped operand), loads the copy
as a separate module and runs a battery of pin checks against it. The battery
uses only independent references: torch's SDPA, the hand-derived worked
example, the pages' layout examples and ring figure, and the exactness claim.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.fp64 as good

SRC_PATH = good.__file__
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_mutant(old: str, new: str):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _check_sdpa(m):
    for (B, Hq, Hkv, S, D, causal) in ((1, 2, 2, 24, 8, True), (1, 4, 2, 20, 8, True),
                                       (1, 2, 2, 16, 8, False)):
        q, k, v = _rand((B, Hq, S, D), 1), _rand((B, Hkv, S, D), 2), _rand((B, Hkv, S, D), 3)
        out, lse = m.attention(q, k, v, causal=causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        g = Hq // Hkv
        tk, tv = tk.repeat_interleave(g, 1), tv.repeat_interleave(g, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal).numpy()
        s = (tq @ tk.transpose(-1, -2)) / math.sqrt(D)
        if causal:
            s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf)
        np.testing.assert_allclose(out, ref, atol=1e-10)
        np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-10)


def _check_hand(m):
    with open(os.path.join(GOLDEN, "hand_case_causal_s3.json")) as f:
        fx = json.load(f)
    q, k, v = (np.array(fx[n])[None, None] for n in ("q", "k", "v"))
    out, lse = m.attention(q, k, v, causal=True, scale=1.0)
    np.testing.assert_allclose(out[0, 0], np.array(fx["out"]), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(fx["lse"]), atol=1e-12)


def _check_layouts(m):
    with open(os.path.join(GOLDEN, "layouts.json")) as f:
        fx = json.load(f)
    for r, exp in enumerate(fx["zigzag_S16_N4_rank_positions"]):
        assert list(m.rank_positions(16, 4, "zigzag", r)) == exp
    order = m.zigzag_order(64, 4)
    assert sorted(order.tolist()) == list(range(64))
    for r, exp in enumerate(fx["striped_S16_N4_rank_positions"]):
        assert list(m.rank_positions(16, 4, "striped", r)) == exp


def _check_schedule(m):
    with open(os.path.join(GOLDEN, "ring_schedule_4gpu.json")) as f:
        fx = json.load(f)
    s = m.ring_schedule(4)
    assert [[int(s[r, 0]), int(s[r, 1])] for r in range(4)] == fx["source_by_rank_step01"]


def _check_ring_exact(m):
    q, k, v = _rand((1, 2, 32, 8), 4), _rand((1, 1, 32, 8), 5), _rand((1, 1, 32, 8), 6)
    for layout in ("contiguous", "zigzag", "striped"):
        ref = good.attention(q, k, v, causal=True)   # the pinned, unmutated definition
        out, lse = m.ring_attention(q, k, v, N=4, layout=layout, causal=True)
        np.testing.assert_allclose(out, ref[0], atol=1e-10)
        np.testing.assert_allclose(lse, ref[1], atol=1e-10)


def _check_merge(m):
    q = _rand((1, 1, 6, 4), 7)
    k1, v1, k2, v2 = (_rand((1, 1, 5, 4), 8 + i) for i in range(4))
    a = good.attention(q, k1, v1, causal=False)
    b = good.attention(q, k2, v2, causal=False)
    u = good.attention(q, np.concatenate([k1, k2], 2), np.concatenate([v1, v2], 2), causal=False)
    o, l_ = m.merge(*a, *b)
    np.testing.assert_allclose(o, u[0], atol=1e-10)
    np.testing.assert_allclose(l_, u[1], atol=1e-10)


BATTERY = (_check_sdpa, _check_hand, _check_layouts, _check_schedule, _check_ring_exact,
           _check_merge)

MUTATIONS = {
    "causal_exclusive": ("allowed = k_pos[None, :] <= q_pos[idx][:, None]",
                         "allowed = k_pos[None, :] < q_pos[idx][:, None]"),
    "dropped_scale": ("s = scale * (q[b, h, idx] @ k[b, g].T)", "s = (q[b, h, idx] @ k[b, g].T)"),
    "wrong_kv_head": ("s = scale * (q[b, h, idx] @ k[b, g].T)",
                      "s = scale * (q[b, h, idx] @ k[b, h % k.shape[1]].T)"),
    "lse_drops_max": ("lse_blk[ok] = m[ok] + np.log(", "lse_blk[ok] = np.log("),
    "out_unnormalised": ("p[ok] = np.exp(s[ok] - lse_blk[ok, None])",
                         "p[ok] = np.exp(s[ok] - m[ok, None])"),
    "out_uses_keys": ("out[b, h, r0:r0 + len(idx)] = p @ v[b, g]",
                      "out[b, h, r0:r0 + len(idx)] = p @ k[b, g]"),
    "zigzag_late_first": ("for chunk in (i, 2 * N - 1 - i):", "for chunk in (2 * N - 1 - i, i):"),
    "zigzag_wrong_pair": ("for chunk in (i, 2 * N - 1 - i):", "for chunk in (i, 2 * N - 2 - i):"),
    "ring_direction": ("return (rank - step) % N", "return (rank + step) % N"),
    "striped_rank_offset": ("if t % N == r:", "if (t + 1) % N == r:"),
    "update_drops_rescale": ("l_new = l_prev * a + l_blk * b", "l_new = l_prev * a + l_blk"),
    "update_sign": ("a = np.where(m_prev > NEG_INF, np.exp(m_prev - m_ref), 0.0)",
                    "a = np.where(m_prev > NEG_INF, np.exp(m_ref - m_prev), 0.0)"),
    "ring_local_mask": ("s = np.where(k_rows[None, :] <= q_rows[:, None], s,",
                        "s = np.where(np.arange(C)[None, :] <= np.arange(C)[:, None], s,"),
    "merge_lse_drops_max": ("lse = np.where(l_new > 0, m_new + np.log(",
                            "lse = np.where(l_new > 0, 0.0 + np.log("),
}


def test_unmutated_oracle_passes_battery():
    for check in BATTERY:
        check(good)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    mutant = _load_mutant(old, new)
    caught = []
    for check in BATTERY:
        try:
            check(mutant)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutation {name} slipped past every pin"
