"""Host-side failure handling and resume of the ring step, on the GPU.

* Watchdog: ra_stream_wait bounds the host's wait for a stream. A stream kept
  busy by ~0.2 s or more of attention work must report RA_ERR_TIMEOUT to a
  10 ms wait, leave that work running undisturbed, and drain under a long
  limit. The stall is real work that ends by itself: nothing here blocks a
  stream for good.
* Checkpoint / resume: the whole state of a rank after k ring steps is its
  fp32 running (out, lse) plus the next step index. Stopping after k steps,
  moving that state to host memory, restoring it into fresh device buffers
  and running the remaining steps must give bit-for-bit the uninterrupted
  result, which must equal exact attention within the bf16 tolerance.
"""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL_BF16, compare

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_context_parallelism_flash_amd")
DEV = "cuda"


def test_stream_wait_times_out_on_a_busy_stream_then_drains():
    B, Hq, Hkv, C, D = 1, 64, 8, 16384, 128
    q = workloads.make_random((B, Hq, C, D), 901, torch.bfloat16).to(DEV)
    k = workloads.make_random((B, Hkv, C, D), 902, torch.bfloat16).to(DEV)
    v = workloads.make_random((B, Hkv, C, D), 903, torch.bfloat16).to(DEV)
    out = torch.empty(B, Hq, C, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, C, dtype=torch.float32, device=DEV)
    ref_out, ref_lse = torch.empty_like(out), torch.empty_like(lse)
    ws = torch.empty(ra.ra_block_attn_workspace_bytes(B, Hkv, C, D, ra.RA_BF16),
                     dtype=torch.uint8, device=DEV)
    ra.ra_block_attn_fwd(q, k, v, ref_out, ref_lse, causal=False, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    ra.ra_stream_wait(s, timeout_ms=1000)  # an idle stream drains at once
    # 40 full 16k x 16k blocks of 64 heads: 3.5e14 flops, 0.2 s or more
    for _ in range(40):
        ra.ra_block_attn_fwd(q, k, v, out, lse, causal=False, workspace=ws, stream=s)
    t0 = time.perf_counter()
    with pytest.raises(ra.RAError) as exc:
        ra.ra_stream_wait(s, timeout_ms=10)
    waited = time.perf_counter() - t0
    print(f"  timed out after {waited * 1e3:.1f} ms: {exc.value}", flush=True)
    assert exc.value.status == ra.RA_ERR_TIMEOUT
    assert 0.010 <= waited < 0.5
    assert not s.query(), "the work must still be running after the timeout"
    ra.ra_stream_wait(s, timeout_ms=60000)
    assert s.query()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def _zigzag_rows(S, N, r):
    c = S // (2 * N)
    return np.concatenate([np.arange(r * c, (r + 1) * c),
                           np.arange((2 * N - 1 - r) * c, (2 * N - r) * c)])


@pytest.mark.parametrize("stop", [1, 3])
def test_ring_resumes_bit_identically_from_a_host_checkpoint(stop):
    B, Hq, Hkv, S, D, N = 1, 4, 2, 2048, 128, 4
    c = S // (2 * N)
    q = workloads.make_random((B, Hq, S, D), 911, torch.bfloat16)
    k = workloads.make_random((B, Hkv, S, D), 912, torch.bfloat16)
    v = workloads.make_random((B, Hkv, S, D), 913, torch.bfloat16)
    rows = [torch.from_numpy(_zigzag_rows(S, N, r)) for r in range(N)]
    qr = [q[:, :, rows[r]].contiguous().to(DEV) for r in range(N)]
    kr = [k[:, :, rows[r]].contiguous().to(DEV) for r in range(N)]
    vr = [v[:, :, rows[r]].contiguous().to(DEV) for r in range(N)]
    pos = [(2, c, r * c, (2 * N - 1 - r) * c) for r in range(N)]

    def steps(r, out, lse, first, last):
        for t in range(first, last):
            src = (r - t) % N
            ra.ra_block_attn_fwd(qr[r], kr[src], vr[src], out, lse, q_pos=pos[r],
                                 k_pos=pos[src], causal=True, accumulate=t > 0)

    def fresh(r):
        return (torch.empty(B, Hq, 2 * c, D, dtype=torch.float32, device=DEV),
                torch.empty(B, Hq, 2 * c, dtype=torch.float32, device=DEV))

    full, resumed = [], []
    for r in range(N):
        out, lse = fresh(r)
        steps(r, out, lse, 0, N)
        full.append((out, lse))
        out, lse = fresh(r)
        steps(r, out, lse, 0, stop)
        torch.cuda.synchronize()
        ckpt = (out.cpu(), lse.cpu(), stop)  # the whole state of the rank
        del out, lse
        out, lse = (ckpt[0].to(DEV), ckpt[1].to(DEV))
        steps(r, out, lse, ckpt[2], N)
        resumed.append((out, lse))
    torch.cuda.synchronize()
    for r in range(N):
        assert torch.equal(full[r][0], resumed[r][0]), f"rank {r}: out differs"
        assert torch.equal(full[r][1], resumed[r][1]), f"rank {r}: lse differs"
    # and the resumed ring is exact attention
    out = np.zeros((B, Hq, S, D))
    lse = np.zeros((B, Hq, S))
    for r in range(N):
        out[:, :, rows[r].numpy()] = resumed[r][0].cpu().double().numpy()
        lse[:, :, rows[r].numpy()] = resumed[r][1].cpu().double().numpy()
    ref_out, ref_lse = oracle.attention(q, k, v, causal=True)
    compare(out, lse, ref_out, ref_lse, TOL_BF16, f"resume after {stop} of {N} steps")
