"""CPU checks of the parity helpers the GPU tests rely on: the rows a large
configuration is checked on, and the process-pool drivers of the oracle
(which must return exactly what a direct oracle call returns)."""
import numpy as np
import pytest

import oracle
from parity_util import GROUP_ROWS, boundary_rows, check_rows, pooled_attention, pooled_backward


def test_check_rows_keeps_every_boundary_row_on_every_head():
    S, Hq, n, chunks = 131072, 64, 4096, 16
    rows = check_rows(S, Hq, n, 3, chunks)
    b = boundary_rows(S, chunks)
    assert rows.shape == (Hq, len(b) + n)
    for h in range(Hq):
        assert np.all(np.diff(rows[h]) > 0)            # sorted, distinct
        assert np.all(np.isin(b, rows[h]))              # every chunk's first and last row
        assert rows[h, 0] == 0 and rows[h, -1] == S - 1
    # the random part is seeded per head: heads differ, reruns agree
    assert not np.array_equal(rows[0], rows[1])
    assert np.array_equal(rows, check_rows(S, Hq, n, 3, chunks))


def test_check_rows_extra_fixed_and_saturation():
    rows = check_rows(64, 2, 100, 0, 4, fixed=[5, 6])
    assert rows.shape == (2, 64)                        # capped at every row
    assert np.array_equal(rows[0], np.arange(64))
    rows = check_rows(1000, 3, 10, 1, 4, fixed=[7])
    assert all(7 in r and 999 in r and 250 in r and 249 in r for r in rows)


@pytest.mark.parametrize("causal", [True, False])
def test_pooled_attention_equals_direct_oracle(causal):
    rng = np.random.default_rng(0)
    Hq, Hkv, S, D = 4, 2, 3 * GROUP_ROWS + 17, 16
    q = rng.standard_normal((1, Hq, S, D)).astype(np.float32)
    k = rng.standard_normal((1, Hkv, S, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, S, D)).astype(np.float32)
    rows = check_rows(S, Hq, 150, 9, 4)
    out, lse = pooled_attention(q, k, v, causal=causal, rows=rows, n_workers=2)
    ref_out, ref_lse = oracle.attention(q, k, v, causal=causal, rows=rows)
    np.testing.assert_allclose(out, ref_out[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse[0], rtol=0, atol=1e-12)


def test_pooled_backward_equals_direct_oracle():
    rng = np.random.default_rng(1)
    Hq, Hkv, S, D, L = 4, 2, 300, 16, 40
    q, dout = (rng.standard_normal((1, Hq, S, D)).astype(np.float32) for _ in range(2))
    k, v = (rng.standard_normal((1, Hkv, S, D)).astype(np.float32) for _ in range(2))
    rows = check_rows(S, Hq, 50, 2, 4, fixed=np.arange(S - L, S))
    dq, dk, dv = pooled_backward(q, k, v, dout, rows=rows, key0=S - L, n_workers=2)
    ref_dq, ref_dk, ref_dv = oracle.attention_backward(q, k, v, dout, causal=True)
    for h in range(Hq):
        np.testing.assert_allclose(dq[h], ref_dq[0, h, rows[h]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, ref_dk[0, :, S - L:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, ref_dv[0, :, S - L:], rtol=0, atol=1e-12)
