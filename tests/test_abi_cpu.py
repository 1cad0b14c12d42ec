"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, reports sizes, and rejects bad arguments on the host before
it touches the HIP runtime."""
import ctypes
import os
import re

import pytest

import ring_context_parallelism_flash_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")

BF16, F32 = ra.RA_BF16, ra.RA_F32
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails validation
FAKE_ODD = ctypes.c_void_p(0x10008)  # 8-byte aligned only


def _declared():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_library_builds_and_loads():
    assert os.path.exists(ra.library_path), "run __graft_entry__.build() first"
    ra.lib()


def test_every_declared_symbol_is_exported():
    declared = _declared()
    assert len(declared) >= 10
    assert sorted(ra.EXPORTS) == declared
    lib = ctypes.CDLL(ra.library_path)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    names = [ra.ra_status_str(s) for s in range(10)]
    assert names == ["RA_OK", "RA_ERR_NULL", "RA_ERR_SHAPE", "RA_ERR_DTYPE", "RA_ERR_UNSUPPORTED",
                     "RA_ERR_ALIGN", "RA_ERR_WORKSPACE", "RA_ERR_ARG", "RA_ERR_HIP",
                     "RA_ERR_TIMEOUT"]


def test_workspace_sizes():
    # bf16 block: V^T padded to 64 keys
    assert ra.ra_block_attn_workspace_bytes(1, 8, 100, 128, BF16) == 1 * 8 * 128 * 128 * 2
    assert ra.ra_block_attn_workspace_bytes(1, 8, 100, 128, F32) == 0
    # ring at the 128k GQA shape: V^T home + 2 slots (K + V^T) + fp32 running out
    C = 131072 // 8
    expect = 8 * 8 * 128 * C * 2 + 2 * (8 * C * 128 * 2 + 8 * 128 * C * 2) + 64 * C * 128 * 4
    assert ra.ra_ring_sim_workspace_bytes(1, 64, 8, 131072, 128, BF16, 8) == expect
    assert ra.ra_ring_sim_workspace_bytes(1, 64, 8, 131071, 128, BF16, 8) == 0  # S % N != 0


def _block(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=1, Hq=2, Hkv=2, Cq=128, Ck=128, D=64,
             dt=F32, qp=None, kp=None, kvmap=None, causal=1, scale=0.125, acc=0, ws=None, wsb=0)
    a.update(kw)
    return ra.lib().ra_block_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                      a["Hkv"], a["Cq"], a["Ck"], a["D"], a["dt"], a["qp"],
                                      a["kp"], a["kvmap"], a["causal"], a["scale"], a["acc"],
                                      a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), "RA_ERR_UNSUPPORTED"),
    (dict(dt=7), "RA_ERR_DTYPE"),
    (dict(Hq=3, Hkv=2), "RA_ERR_SHAPE"),
    (dict(B=0), "RA_ERR_SHAPE"),
    (dict(Cq=-1), "RA_ERR_SHAPE"),
    (dict(scale=0.0), "RA_ERR_ARG"),
    (dict(scale=float("nan")), "RA_ERR_ARG"),
    (dict(causal=2), "RA_ERR_ARG"),
    (dict(q=None), "RA_ERR_NULL"),
    (dict(k=None), "RA_ERR_NULL"),
    (dict(out=FAKE_ODD), "RA_ERR_ALIGN"),
    (dict(dt=BF16), "RA_ERR_WORKSPACE"),
    (dict(dt=BF16, ws=FAKE, wsb=10), "RA_ERR_WORKSPACE"),
    (dict(Hq=300, Hkv=300), "RA_ERR_UNSUPPORTED"),
])
def test_block_attn_rejects(kw, status):
    st = _block(**kw)
    assert ra.ra_status_str(st) == status, ra.ra_last_error()
    assert ra.ra_last_error() != ""


def test_block_attn_rejects_bad_positions_and_map():
    bad = [ra.ra_pos(3, 128, (ctypes.c_int64 * 2)(0, 0)),        # nseg
           ra.ra_pos(2, 60, (ctypes.c_int64 * 2)(0, 100)),       # 2*60 != 128
           ra.ra_pos(2, 64, (ctypes.c_int64 * 2)(0, 10)),        # overlapping segments
           ra.ra_pos(1, 128, (ctypes.c_int64 * 2)(-5, 0)),       # negative start
           ra.ra_pos(1, 128, (ctypes.c_int64 * 2)(0, 0), -2),    # negative stride
           ra.ra_pos(2, 64, (ctypes.c_int64 * 2)(0, 120), 2)]    # stride-2 segment 0 ends at 126
    for p in bad:
        assert ra.ra_status_str(_block(qp=ctypes.byref(p))) == "RA_ERR_SHAPE"
    far = ra.ra_pos(1, 128, (ctypes.c_int64 * 2)(0, 0), 1 << 25)    # last position 127 * 2^25
    assert ra.ra_status_str(_block(kp=ctypes.byref(far))) == "RA_ERR_UNSUPPORTED"
    ok = [ra.ra_pos(2, 64, (ctypes.c_int64 * 2)(0, 127), 2),         # segment 0 ends at 126
          ra.ra_pos(1, 128, (ctypes.c_int64 * 2)(3, 0), 0)]         # stride 0 reads as 1
    for p in ok:   # valid positions: the call gets as far as the workspace check
        assert ra.ra_status_str(_block(qp=ctypes.byref(p), dt=BF16)) == "RA_ERR_WORKSPACE"
    m = (ctypes.c_int32 * 2)(0, 2)  # kv head 2 of 2
    assert ra.ra_status_str(_block(kvmap=m)) == "RA_ERR_SHAPE"


def test_empty_query_block_is_a_no_op():
    assert _block(Cq=0, q=None, out=None, lse=None) == 0


def test_ring_rejects():
    L = ra.lib()

    def ring(**kw):
        a = dict(S=1024, N=4, layout=1, dt=BF16, ws=None, wsb=0, D=128, Hq=8, Hkv=2)
        a.update(kw)
        return ra.ra_status_str(L.ra_ring_sim_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, a["Hq"], a["Hkv"],
                                                  a["S"], a["D"], a["dt"], a["N"], a["layout"], 1,
                                                  0.088, None, a["ws"], a["wsb"], None, None))
    assert ring(S=1020) == "RA_ERR_SHAPE"         # divisible by N=4 but not by 2N (zigzag)
    assert ring(S=1028, layout=0) == "RA_ERR_WORKSPACE"  # divisible by N: ok until workspace
    assert ring(N=0) == "RA_ERR_SHAPE"
    assert ring(layout=5) == "RA_ERR_ARG"
    assert ring(S=1020, layout=2) == "RA_ERR_WORKSPACE"  # striped: divisible by N suffices
    assert ring() == "RA_ERR_WORKSPACE"
    assert ring(S=0) == "RA_OK"


def test_permute_and_merge_reject():
    L = ra.lib()
    assert ra.ra_status_str(L.ra_zigzag_permute(FAKE, FAKE, 1, 1000, 2, 8, 0, None)) == "RA_ERR_SHAPE"
    assert ra.ra_status_str(L.ra_zigzag_permute(FAKE, FAKE, 1, 1024, 2, 8, 0, None)) == "RA_ERR_ARG"
    assert ra.ra_status_str(L.ra_zigzag_permute(None, FAKE, 1, 1024, 2, 8, 0, None)) == "RA_ERR_NULL"
    assert ra.ra_status_str(L.ra_zigzag_permute(FAKE, FAKE, 1, 1024, 2, 8, 3, None)) == "RA_ERR_ARG"
    assert ra.ra_status_str(L.ra_striped_permute(FAKE, FAKE, 1, 1001, 2, 8, 0, None)) == "RA_ERR_SHAPE"
    assert ra.ra_status_str(L.ra_striped_permute(FAKE, FAKE, 1, 1000, 2, 8, 0, None)) == "RA_ERR_ARG"
    assert ra.ra_status_str(L.ra_striped_permute(None, FAKE, 1, 1000, 2, 8, 0, None)) == "RA_ERR_NULL"
    assert ra.ra_status_str(L.ra_striped_permute(FAKE, FAKE, 1, 1000, 2, 0, 0, None)) == "RA_ERR_SHAPE"
    assert L.ra_striped_permute(None, None, 0, 1000, 2, 8, 0, None) == 0
    assert ra.ra_status_str(L.ra_lse_merge(None, FAKE, FAKE, FAKE, 10, 4, None)) == "RA_ERR_NULL"
    assert ra.ra_status_str(L.ra_lse_merge(FAKE, FAKE, FAKE, FAKE, 10, 0, None)) == "RA_ERR_SHAPE"
    assert L.ra_lse_merge(None, None, None, None, 0, 4, None) == 0


def test_backward_workspace_sizes_and_rejects():
    L = ra.lib()
    assert ra.ra_block_attn_bwd_workspace_bytes(1, 8, 2, 300, 200, 128, F32) == 0   # bf16 only
    n = ra.ra_block_attn_bwd_workspace_bytes(1, 8, 2, 300, 200, 128, BF16)
    # Q^T, dO^T [8][128][384] bf16 + K^T [2][128][256] bf16 + two [8][384] fp32 rows
    assert n == 2 * 8 * 128 * 384 * 2 + 2 * 128 * 256 * 2 + 2 * 8 * 384 * 4
    assert ra.ra_ring_sim_bwd_workspace_bytes(1, 8, 2, 1000, 128, BF16, 3) == 0     # S % N
    assert ra.ra_ring_sim_bwd_workspace_bytes(1, 8, 2, 1024, 128, BF16, 4) > 0

    def block(**kw):
        a = dict(dt=BF16, D=128, Hq=2, Hkv=2, Cq=64, Ck=64, q=FAKE, dq=FAKE, ws=None, wsb=0,
                 causal=1)
        a.update(kw)
        return ra.ra_status_str(L.ra_block_attn_bwd(
            a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, a["dq"], FAKE, FAKE, 1, a["Hq"], a["Hkv"],
            a["Cq"], a["Ck"], a["D"], a["dt"], None, None, None, a["causal"], 0.088, a["ws"],
            a["wsb"], None))
    assert block(dt=F32) == "RA_ERR_UNSUPPORTED"
    assert block(D=96) == "RA_ERR_UNSUPPORTED"
    assert block(Hq=3) == "RA_ERR_SHAPE"
    assert block(q=None) == "RA_ERR_NULL"
    assert block(dq=FAKE_ODD) == "RA_ERR_ALIGN"
    assert block(causal=3) == "RA_ERR_ARG"
    assert block() == "RA_ERR_WORKSPACE"
    assert block(Cq=0) == "RA_OK" and block(Ck=0) == "RA_OK"

    def ring(**kw):
        a = dict(dt=BF16, S=1024, N=4, layout=1)
        a.update(kw)
        return ra.ra_status_str(L.ra_ring_sim_bwd(
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, a["S"], 128, a["dt"],
            a["N"], a["layout"], 1, 0.088, None, None, 0, None))
    assert ring(dt=F32) == "RA_ERR_UNSUPPORTED"
    assert ring(S=1020) == "RA_ERR_SHAPE"
    assert ring(layout=9) == "RA_ERR_ARG"
    assert ring(S=1020, layout=2) == "RA_ERR_WORKSPACE"
    assert ring() == "RA_ERR_WORKSPACE"
    assert ring(S=0) == "RA_OK"


def test_ulysses_workspace_sizes_and_rejects():
    L = ra.lib()
    # head-sharded q, out [8][1000][128] and k, v [4][1000][128], + V^T [4][128][1024] (bf16)
    assert ra.ra_ulysses_sim_workspace_bytes(1, 8, 4, 1000, 128, BF16, 4) == \
        2 * (8 * 1000 * 128 * 2) + 2 * (4 * 1000 * 128 * 2) + 4 * 128 * 1024 * 2
    assert ra.ra_ulysses_sim_workspace_bytes(1, 8, 4, 1000, 128, F32, 4) == \
        2 * (8 * 1000 * 128 * 4) + 2 * (4 * 1000 * 128 * 4)
    assert ra.ra_ulysses_sim_workspace_bytes(1, 8, 4, 1001, 128, BF16, 4) == 0     # S % P

    def sim(**kw):
        a = dict(dt=BF16, D=128, Hq=8, Hkv=4, S=1024, P=4, q=FAKE, out=FAKE, causal=1, kv=None)
        a.update(kw)
        kv = None if a["kv"] is None else (ctypes.c_int32 * len(a["kv"]))(*a["kv"])
        return ra.ra_status_str(L.ra_ulysses_sim_fwd(
            a["q"], FAKE, FAKE, a["out"], FAKE, 1, a["Hq"], a["Hkv"], a["S"], a["D"], a["dt"],
            a["P"], a["causal"], 0.088, kv, None, 0, None))
    assert sim(D=96) == "RA_ERR_UNSUPPORTED"
    assert sim(P=8) == "RA_ERR_SHAPE"                      # P > H_KV
    assert sim(P=3) == "RA_ERR_SHAPE"                      # heads not divisible by P
    assert sim(S=1022) == "RA_ERR_SHAPE"                   # S % P
    assert sim(kv=[2, 2, 0, 0, 1, 1, 3, 3]) == "RA_ERR_SHAPE"   # head 0 reads rank 1's KV head
    assert sim(kv=[1, 0, 1, 0, 3, 3, 2, 2], P=2) == "RA_ERR_WORKSPACE"  # rank-local map: fine
    assert sim(causal=2) == "RA_ERR_ARG"
    assert sim(q=None) == "RA_ERR_NULL"
    assert sim(out=FAKE_ODD) == "RA_ERR_ALIGN"
    assert sim() == "RA_ERR_WORKSPACE"
    assert sim(S=0) == "RA_OK"

    def a2a(src=FAKE, dst=ctypes.c_void_p(0x7000000), B=1, S=1024, H=8, P=4, inv=0):
        return ra.ra_status_str(L.ra_ulysses_all_to_all(src, dst, B, S, H, 256, P, inv, None))
    assert a2a(S=1022) == "RA_ERR_SHAPE"
    assert a2a(H=6) == "RA_ERR_SHAPE"
    assert a2a(P=0) == "RA_ERR_SHAPE"
    assert a2a(inv=2) == "RA_ERR_ARG"
    assert a2a(src=None) == "RA_ERR_NULL"
    assert a2a(dst=ctypes.c_void_p(0x10000 + 4096)) == "RA_ERR_ARG"    # overlap
    assert a2a(B=0) == "RA_OK" and a2a(S=0) == "RA_OK"


def test_usp_workspace_sizes_and_rejects():
    L = ra.lib()
    ring = ra.ra_ring_sim_workspace_bytes(1, 4, 2, 1024, 128, BF16, 4)
    up = lambda x: (x + 255) // 256 * 256
    # head-sharded q, out [8][1024][128] and k, v [4][1024][128] bf16, + one ring workspace
    assert ra.ra_usp_sim_workspace_bytes(1, 8, 4, 1024, 128, BF16, 2, 4) == \
        2 * (8 * 1024 * 128 * 2) + 2 * (4 * 1024 * 128 * 2) + up(ring)
    assert ra.ra_usp_sim_workspace_bytes(1, 8, 4, 1020, 128, BF16, 2, 4) == 0    # S % (P_u*P_r)

    def usp(**kw):
        a = dict(S=1024, P_u=2, P_r=4, layout=1, Hq=8, Hkv=4, kv=None)
        a.update(kw)
        kv = None if a["kv"] is None else (ctypes.c_int32 * len(a["kv"]))(*a["kv"])
        return ra.ra_status_str(L.ra_usp_sim_fwd(
            FAKE, FAKE, FAKE, FAKE, FAKE, 1, a["Hq"], a["Hkv"], a["S"], 128, BF16, a["P_u"],
            a["P_r"], a["layout"], 1, 0.088, kv, None, 0, None, None))
    assert usp(P_u=8) == "RA_ERR_SHAPE"                 # P_u > H_KV
    assert usp(S=1004) == "RA_ERR_SHAPE"                # S % (P_u * P_r)
    assert usp(S=1029, P_r=3, P_u=1) == "RA_ERR_SHAPE"  # zigzag: S % (2 P_r)
    assert usp(layout=7) == "RA_ERR_ARG"
    assert usp(kv=[2, 2, 0, 0, 1, 1, 3, 3]) == "RA_ERR_SHAPE"
    assert usp() == "RA_ERR_WORKSPACE"
    assert usp(S=0) == "RA_OK"


def test_timing_read_without_launches():
    ra.ra_kernel_timing_enable(True)
    ms, n, fl = ra.ra_kernel_timing_read()
    ra.ra_kernel_timing_enable(False)
    assert (ms, n, fl) == (0.0, 0, 0.0)


def test_no_cpu_fallback_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(ra, "_lib", None)
    monkeypatch.setattr(ra, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(ra.RAError):
        ra.lib()


def test_stream_wait_rejects_a_negative_timeout_before_any_hip_call():
    assert ra.ra_status_str(ra.lib().ra_stream_wait(None, -1)) == "RA_ERR_ARG"
    assert "timeout_ms" in ra.ra_last_error()
