"""GPU test of ra_block_attn_fwd_noalloc, the entry point for callers that
cannot allocate device memory: through the C ABI, two calls in a row (the
second smaller) must give bit-for-bit the result of ra_block_attn_fwd with a
caller workspace (the same kernels), and match the fp64 oracle within the
bf16 tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL_BF16, compare

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_context_parallelism_flash_amd")
DEV = "cuda"


def _pos_array(desc, rows):
    nseg, seg, *rest = desc
    rest = list(rest) + [0] * (3 - len(rest))
    s0, s1 = rest[0], rest[1]
    t = np.arange(rows)
    return s0 + t if nseg == 1 else np.where(t < seg, s0 + t, s1 + (t - seg))


def _one(Hq, Hkv, Cq, Ck, q_pos, k_pos, accumulate, seed):
    D = 128
    q = workloads.make_random((1, Hq, Cq, D), seed, torch.bfloat16)
    k = workloads.make_random((1, Hkv, Ck, D), seed + 1, torch.bfloat16)
    v = workloads.make_random((1, Hkv, Ck, D), seed + 2, torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if accumulate:
        out0 = torch.zeros(1, Hq, Cq, D)
        lse0 = torch.full((1, Hq, Cq), -float("inf"))
        lse0[..., ::3] = 1.5         # some rows carry an earlier state
        out0[..., ::3, :] = workloads.make_random((1, Hq, (Cq + 2) // 3, D), seed + 3)
    else:
        out0 = torch.full((1, Hq, Cq, D), 7.0)    # garbage: overwritten
        lse0 = torch.full((1, Hq, Cq), 3.0)
    o1, l1 = out0.to(DEV), lse0.to(DEV)
    o2, l2 = out0.to(DEV), lse0.to(DEV)
    args = dict(q_pos=q_pos, k_pos=k_pos, causal=True, accumulate=accumulate)
    ra.ra_block_attn_fwd(qd, kd, vd, o1, l1, **args)
    ra.ra_block_attn_fwd_noalloc(qd, kd, vd, o2, l2, **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    qp, kp = _pos_array(q_pos, Cq), _pos_array(k_pos, Ck)
    ref_out, ref_lse = oracle.attention(q, k, v, causal=True, q_pos=qp, k_pos=kp)
    if accumulate:
        ref_out, ref_lse = oracle.merge(out0, lse0, ref_out, ref_lse)
    compare(o2.double().cpu().numpy(), l2.double().cpu().numpy(), ref_out, ref_lse, TOL_BF16,
            f"noalloc Hq={Hq} Hkv={Hkv} Cq={Cq} Ck={Ck} acc={accumulate}")


def test_noalloc_two_calls_match_workspace_entry_point_and_oracle():
    # 32 MiB of transposed V (8 KV heads x 16384 keys): a diagonal across the block
    _one(Hq=8, Hkv=8, Cq=300, Ck=16384, q_pos=(1, 300, 16000), k_pos=(1, 16384, 0),
         accumulate=False, seed=301)
    # then a smaller, ragged GQA block on two position segments, accumulating
    _one(Hq=4, Hkv=2, Cq=384, Ck=1000, q_pos=(2, 192, 100, 1500), k_pos=(2, 500, 0, 1200),
         accumulate=True, seed=311)


def test_noalloc_rejects_blocks_beyond_the_scratch():
    """8 KV heads x 40000 keys x 128 x 2 bytes exceeds 64 MiB: RA_ERR_WORKSPACE,
    decided on the host before anything is enqueued."""
    q = torch.zeros(1, 8, 64, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 8, 40000, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(1, 8, 64, 128, device=DEV)
    lse = torch.zeros(1, 8, 64, device=DEV)
    with pytest.raises(ra.RAError) as ei:
        ra.ra_block_attn_fwd_noalloc(q, k, k, out, lse, causal=False)
    assert ei.value.status == 6 and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == 0)
