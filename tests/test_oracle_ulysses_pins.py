"""Pins for the fp64 Ulysses oracle (CPU only), independent of its own code.

  fixture   -- the hand-worked P=2 all-to-all in tests/golden/ulysses_a2a.json
  labels    -- every element, labelled with its (batch, position, head, dim),
               lands where the page's layouts say: rank j, row t, head
               j*H/P + h' (and back)
  exact     -- Ulysses attention equals single-device attention [the result
               is that of one device], causal and not, MHA and GQA
  volume    -- the count of elements that change rank equals the page's
               (P-1)/P * b*s*h
  limits    -- H divisible by P; P <= H_KV under GQA (8 KV heads: at most 8)
  mutation  -- planted mistakes in a copy of the oracle are caught
"""
import json
import pathlib
import types

import numpy as np
import pytest

import oracle
import oracle.fp64_ulysses as good

GOLDEN = pathlib.Path(__file__).parent / "golden" / "ulysses_a2a.json"


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _shard(x, P):
    """[B, H, S, D] in sequence order -> the ranks' slices [P, B, S/P, H, D]."""
    B, H, S, D = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, P, S // P, H, D).transpose(1, 0, 2, 3, 4)


def _unshard(x):
    """[P, B, S/P, H, D] -> [B, H, S, D]."""
    P, B, Sp, H, D = x.shape
    return x.transpose(1, 0, 2, 3, 4).reshape(B, P * Sp, H, D).transpose(0, 2, 1, 3)


# ------------------------------------------------------------------- fixture
def test_golden_fixture():
    g = json.loads(GOLDEN.read_text())
    x = np.array(g["input_per_rank_S_by_H"], dtype=np.float64)[:, None, :, :, None]
    y = oracle.ulysses_all_to_all(x, g["P"])
    np.testing.assert_array_equal(y[:, 0, :, :, 0], np.array(g["after_all_to_all_per_rank_S_by_Hp"]))
    np.testing.assert_array_equal(oracle.ulysses_all_to_all_inverse(y, g["P"]), x)
    assert oracle.ulysses_volume(1, 4, 4, 1, 2) == g["volume_elements"]


# -------------------------------------------------------------------- labels
def _labels(P, B, S, H, D):
    """x[p, b, i, h, d] = code of (b, global position p*S/P + i, h, d)."""
    Sp = S // P
    p, b, i, h, d = np.meshgrid(np.arange(P), np.arange(B), np.arange(Sp), np.arange(H),
                                np.arange(D), indexing="ij")
    return (((b * S + p * Sp + i) * H + h) * D + d).astype(np.int64)


@pytest.mark.parametrize("P,B,S,H,D", [(2, 1, 4, 4, 1), (4, 2, 12, 8, 3), (8, 1, 16, 8, 2),
                                       (1, 2, 6, 3, 2), (3, 1, 9, 6, 1)])
def test_labels_land_where_the_layouts_say(P, B, S, H, D):
    x = _labels(P, B, S, H, D)
    y = oracle.ulysses_all_to_all(x, P)
    Hp = H // P
    j, b, t, hh, d = np.meshgrid(np.arange(P), np.arange(B), np.arange(S), np.arange(Hp),
                                 np.arange(D), indexing="ij")
    expect = ((b * S + t) * H + j * Hp + hh) * D + d     # rank j: heads j*Hp.., every position
    np.testing.assert_array_equal(y, expect)
    np.testing.assert_array_equal(oracle.ulysses_all_to_all_inverse(y, P), x)


# --------------------------------------------------------------------- exact
@pytest.mark.parametrize("P,B,Hq,Hkv,S,D,causal", [
    (2, 1, 4, 2, 16, 8, True), (4, 1, 8, 4, 24, 8, True), (4, 2, 4, 4, 16, 4, False),
    (1, 1, 2, 1, 10, 8, True), (2, 1, 8, 2, 20, 16, True),
])
def test_exact_equals_single_device(P, B, Hq, Hkv, S, D, causal):
    q, k, v = _rand((B, Hq, S, D), 1), _rand((B, Hkv, S, D), 2), _rand((B, Hkv, S, D), 3)
    ref_out, ref_lse = oracle.attention(q, k, v, causal=causal)
    out, lse = oracle.ulysses_attention(_shard(q, P), _shard(k, P), _shard(v, P), P=P, causal=causal)
    np.testing.assert_allclose(_unshard(out), ref_out, atol=1e-12)
    # lse stays head-sharded: rank j holds heads j*Hq/P ..
    np.testing.assert_allclose(lse.transpose(1, 0, 2, 3).reshape(B, Hq, S), ref_lse, atol=1e-12)


def test_exact_with_a_rank_local_kv_map():
    P, Hq, Hkv, S, D = 2, 8, 4, 12, 8
    kv_map = [1, 0, 1, 0, 3, 2, 2, 3]
    q, k, v = _rand((1, Hq, S, D), 4), _rand((1, Hkv, S, D), 5), _rand((1, Hkv, S, D), 6)
    ref_out, _ = oracle.attention(q, k, v, causal=True, kv_head_of_q=kv_map)
    out, _ = oracle.ulysses_attention(_shard(q, P), _shard(k, P), _shard(v, P), P=P, causal=True,
                                      kv_head_of_q=kv_map)
    np.testing.assert_allclose(_unshard(out), ref_out, atol=1e-12)


# -------------------------------------------------------------------- volume
@pytest.mark.parametrize("P,B,S,H,D", [(2, 1, 4, 4, 1), (4, 2, 8, 4, 2), (8, 1, 16, 8, 3),
                                       (1, 1, 4, 2, 2)])
def test_volume_counts_elements_that_change_rank(P, B, S, H, D):
    Sp = S // P
    src_rank = np.broadcast_to(np.arange(P)[:, None, None, None, None], (P, B, Sp, H, D))
    y = oracle.ulysses_all_to_all(src_rank, P)
    moved = int((y != np.arange(P)[:, None, None, None, None]).sum())
    assert moved == oracle.ulysses_volume(B, S, H, D, P)


# -------------------------------------------------------------------- limits
def test_limits():
    q = np.zeros((8, 1, 2, 64, 4))
    kv8 = np.zeros((8, 1, 2, 8, 4))
    oracle.ulysses_attention(q, kv8, kv8, P=8, causal=True)          # 8 KV heads, P = 8: fine
    q16 = np.zeros((16, 1, 1, 64, 4))
    kv16 = np.zeros((16, 1, 1, 8, 4))
    with pytest.raises(ValueError):                                   # P = 16 > 8 KV heads
        oracle.ulysses_attention(q16, kv16, kv16, P=16, causal=True)
    with pytest.raises(ValueError):                                   # H not divisible by P
        oracle.ulysses_all_to_all(np.zeros((4, 1, 2, 6, 1)), 4)
    with pytest.raises(ValueError):                                   # head reads another rank's KV
        oracle.ulysses_attention(np.zeros((2, 1, 2, 4, 2)), np.zeros((2, 1, 2, 2, 2)),
                                 np.zeros((2, 1, 2, 2, 2)), P=2, causal=True,
                                 kv_head_of_q=[1, 1, 0, 0])


# ------------------------------------------------------------------ mutation
def _mutant(old, new):
    src = pathlib.Path(good.__file__).read_text()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_ulysses_mutant")
    mod.__dict__["__package__"] = "oracle"
    mod.__dict__["__name__"] = "oracle.fp64_ulysses_mutant"
    exec(compile(src.replace(old, new), "oracle_ulysses_mutant", "exec"), mod.__dict__)
    return mod


def _battery(m):
    P, Hq, Hkv, S, D = 2, 8, 4, 12, 8
    kv_map = [1, 0, 1, 0, 3, 2, 2, 3]
    q, k, v = _rand((1, Hq, S, D), 7), _rand((1, Hkv, S, D), 8), _rand((1, Hkv, S, D), 9)
    ref_out, ref_lse = oracle.attention(q, k, v, causal=True, kv_head_of_q=kv_map)
    out, lse = m.ulysses_attention(_shard(q, P), _shard(k, P), _shard(v, P), P=P, causal=True,
                                   kv_head_of_q=kv_map)
    np.testing.assert_allclose(_unshard(out), ref_out, atol=1e-12)
    np.testing.assert_allclose(lse.transpose(1, 0, 2, 3).reshape(1, Hq, S), ref_lse, atol=1e-12)
    x = _labels(4, 1, 8, 4, 1)
    y = m.ulysses_all_to_all(x, 4)
    np.testing.assert_array_equal(m.ulysses_all_to_all_inverse(y, 4), x)
    g = json.loads(GOLDEN.read_text())
    gx = np.array(g["input_per_rank_S_by_H"], dtype=np.float64)[:, None, :, :, None]
    np.testing.assert_array_equal(m.ulysses_all_to_all(gx, 2)[:, 0, :, :, 0],
                                  np.array(g["after_all_to_all_per_rank_S_by_Hp"]))
    assert m.ulysses_volume(1, 4, 4, 1, 2) == g["volume_elements"]


MUTATIONS = {
    "a2a_heads_of_sender": ("y[j, :, p * Sp:(p + 1) * Sp] = x[p, :, :, j * Hp:(j + 1) * Hp]",
                            "y[j, :, p * Sp:(p + 1) * Sp] = x[p, :, :, p * Hp:(p + 1) * Hp]"),
    "a2a_offset_of_receiver": ("y[j, :, p * Sp:(p + 1) * Sp] = x[p",
                               "y[j, :, ((p + j) % P) * Sp:((p + j) % P + 1) * Sp] = x[p"),
    "inverse_rows_of_sender": ("= y[j, :, p * Sp:(p + 1) * Sp]", "= y[j, :, j * Sp:(j + 1) * Sp]"),
    "local_map_not_shifted": ("local_map = [kv_map[j * Hqp + h] - j * Hkvp for h in range(Hqp)]",
                              "local_map = [kv_map[h] for h in range(Hqp)]"),
    "volume_per_rank_slice": ("return (P - 1) / P * B * S * H * D",
                              "return (P - 1) / P * B * (S // P) * H * D"),
}


def test_unmutated_ulysses_passes_battery():
    _battery(good)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_ulysses_planted_mistake_is_caught(name):
    m = _mutant(*MUTATIONS[name])
    with pytest.raises(AssertionError):
        _battery(m)


# ====================================================================== USP
USP_GOLDEN = pathlib.Path(__file__).parent / "golden" / "usp_devices.json"


def _usp_shard(x, P_u, P_r, layout):
    """[B, H, S, D] sequence order -> device slices [P_r*P_u, B, S/(P_r*P_u), H, D]."""
    B, H, S, D = x.shape
    L = oracle.usp_token_lists(S, P_r, layout).reshape(-1)
    xs = x[:, :, L].transpose(0, 2, 1, 3)
    return xs.reshape(B, P_r * P_u, S // (P_r * P_u), H, D).transpose(1, 0, 2, 3, 4)


def test_usp_golden_device_positions():
    g = json.loads(USP_GOLDEN.read_text())
    lists = oracle.usp_token_lists(g["S"], g["P_r"], g["layout"])
    np.testing.assert_array_equal(lists, np.array(g["node_token_lists"]))
    pos = np.arange(g["S"], dtype=float)[None, None, :, None]          # value = position
    dev = _usp_shard(pos, g["P_u"], g["P_r"], g["layout"])[:, 0, :, 0, 0]
    np.testing.assert_array_equal(dev, np.array(g["device_positions"]))


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("P_u,P_r,Hq,Hkv,causal", [(2, 4, 4, 2, True), (4, 2, 8, 4, True),
                                                   (2, 2, 4, 2, False), (1, 4, 2, 1, True),
                                                   (4, 1, 4, 4, True)])
def test_usp_exact_equals_single_device(layout, P_u, P_r, Hq, Hkv, causal):
    S, D = 64, 8
    q, k, v = _rand((1, Hq, S, D), 31), _rand((1, Hkv, S, D), 32), _rand((1, Hkv, S, D), 33)
    out, lse = oracle.usp_attention(*(_usp_shard(t, P_u, P_r, layout) for t in (q, k, v)),
                                    P_u=P_u, P_r=P_r, layout=layout, causal=causal)
    ro, rl = oracle.attention(q, k, v, causal=causal)
    L = oracle.usp_token_lists(S, P_r, layout).reshape(-1)
    np.testing.assert_allclose(out, _usp_shard(ro, P_u, P_r, layout), atol=1e-12)
    np.testing.assert_allclose(lse.transpose(1, 0, 2, 3).reshape(1, Hq, S), rl[:, :, L], atol=1e-12)


def test_usp_reduces_to_ulysses_and_to_ring():
    S, D, Hq, Hkv = 48, 8, 4, 2
    q, k, v = _rand((1, Hq, S, D), 34), _rand((1, Hkv, S, D), 35), _rand((1, Hkv, S, D), 36)
    # one node: USP is Ulysses over P_u devices
    uo, ul = oracle.ulysses_attention(_shard(q, 4 // 2), _shard(k, 2), _shard(v, 2), P=2, causal=True)
    so, sl = oracle.usp_attention(_shard(q, 2), _shard(k, 2), _shard(v, 2), P_u=2, P_r=1,
                                  layout="contiguous", causal=True)
    np.testing.assert_allclose(so, uo, atol=1e-12)
    np.testing.assert_allclose(sl, ul, atol=1e-12)
    # one device per node: USP is the ring over P_r ranks (lse in rank-major order)
    ro, rl = oracle.ring_attention(q, k, v, N=4, layout="zigzag", causal=True)
    so, sl = oracle.usp_attention(*(_usp_shard(t, 1, 4, "zigzag") for t in (q, k, v)), P_u=1,
                                  P_r=4, layout="zigzag", causal=True)
    L = oracle.usp_token_lists(S, 4, "zigzag").reshape(-1)
    np.testing.assert_allclose(so, _usp_shard(ro, 1, 4, "zigzag"), atol=1e-12)
    np.testing.assert_allclose(sl[0], rl[:, :, L], atol=1e-12)


def test_usp_degree_limit():
    """The Ulysses dimension is bounded by the KV heads: degree H_KV x nodes."""
    z = lambda *s: np.zeros(s)
    oracle.usp_attention(z(16, 1, 2, 8, 4), z(16, 1, 2, 8, 4), z(16, 1, 2, 8, 4), P_u=8, P_r=2,
                         layout="contiguous", causal=True)
    with pytest.raises(ValueError):
        oracle.usp_attention(z(32, 1, 1, 16, 4), z(32, 1, 1, 8, 4), z(32, 1, 1, 8, 4), P_u=16,
                             P_r=2, layout="contiguous", causal=True)


def _usp_battery(m):
    S, D, Hq, Hkv, P_u, P_r = 32, 8, 8, 4, 2, 2
    kv_map = [1, 0, 1, 0, 3, 2, 2, 3]
    q, k, v = _rand((1, Hq, S, D), 37), _rand((1, Hkv, S, D), 38), _rand((1, Hkv, S, D), 39)
    for layout in ("zigzag", "striped"):
        out, lse = m.usp_attention(*(_usp_shard(t, P_u, P_r, layout) for t in (q, k, v)), P_u=P_u,
                                   P_r=P_r, layout=layout, causal=True, kv_head_of_q=kv_map)
        ro, rl = oracle.attention(q, k, v, causal=True, kv_head_of_q=kv_map)
        L = oracle.usp_token_lists(S, P_r, layout).reshape(-1)
        np.testing.assert_allclose(out, _usp_shard(ro, P_u, P_r, layout), atol=1e-10)
        np.testing.assert_allclose(lse.transpose(1, 0, 2, 3).reshape(1, Hq, S), rl[:, :, L],
                                   atol=1e-10)


USP_MUTATIONS = {
    "a2a_across_nodes": ("ulysses_all_to_all(t[n * P_u:(n + 1) * P_u], P_u)",
                         "ulysses_all_to_all(t[n::P_r], P_u)"),
    "node_order_taken_as_sequence": ("order = lists.reshape(-1)        # node-major position list",
                                     "order = np.arange(S)"),
    "usp_local_map_not_shifted": (
        "        local_map = [kv_map[u * Hqp + h] - u * Hkvp for h in range(Hqp)]\n        # head group u",
        "        local_map = [kv_map[h] for h in range(Hqp)]\n        # head group u"),
    "lse_in_sequence_order": ("lse[u] = l_nm", "lse[u] = l"),
}


def test_unmutated_usp_passes_battery():
    _usp_battery(good)


@pytest.mark.parametrize("name", sorted(USP_MUTATIONS))
def test_usp_planted_mistake_is_caught(name):
    m = _mutant(*USP_MUTATIONS[name])
    with pytest.raises(AssertionError):
        _usp_battery(m)
