"""Python binding of the MI355X ring-attention library (``libringattn.so``).

The functions below carry the C ABI's names and only marshal arguments:
torch tensors provide device memory and ``torch.cuda`` streams provide the
HIP stream handles; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is not built or cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "RAError", "lib", "library_path", "RA_BF16", "RA_F32", "RA_CONTIGUOUS", "RA_ZIGZAG",
    "ra_pos", "ra_status_str", "ra_last_error", "ra_block_attn_workspace_bytes",
    "ra_block_attn_fwd", "ra_block_attn_fwd_noalloc", "ra_lse_merge", "ra_zigzag_permute",
    "ra_striped_permute", "ra_ring_sim_workspace_bytes", "ra_block_attn_bwd_workspace_bytes", "ra_block_attn_bwd",
    "ra_ring_sim_bwd_workspace_bytes", "ra_ring_sim_bwd", "ring_attention_sim_backward",
    "ra_ring_sim_fwd", "ra_kernel_timing_enable", "ra_kernel_timing_read", "ring_attention_sim", "ra_ulysses_all_to_all",
    "ra_ulysses_sim_workspace_bytes", "ra_ulysses_sim_fwd", "ra_usp_sim_workspace_bytes",
    "ra_usp_sim_fwd", "ra_device_info", "ra_mfma_probe_bf16", "ra_stream_wait", "RA_ERR_TIMEOUT",
    "EXPORTS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libringattn.so")

RA_BF16, RA_F32 = 0, 1
RA_CONTIGUOUS, RA_ZIGZAG, RA_STRIPED = 0, 1, 2
RA_ERR_TIMEOUT = 9
_DTYPES = {torch.bfloat16: RA_BF16, torch.float32: RA_F32}
_LAYOUTS = {"contiguous": RA_CONTIGUOUS, "zigzag": RA_ZIGZAG, "striped": RA_STRIPED}

# Every symbol include/ring_attn.h declares.
EXPORTS = (
    "ra_status_str", "ra_last_error", "ra_block_attn_workspace_bytes", "ra_block_attn_fwd",
    "ra_block_attn_fwd_noalloc", "ra_lse_merge", "ra_zigzag_permute", "ra_striped_permute", "ra_ring_sim_workspace_bytes",
    "ra_ring_sim_fwd", "ra_block_attn_bwd_workspace_bytes", "ra_block_attn_bwd",
    "ra_ring_sim_bwd_workspace_bytes", "ra_ring_sim_bwd", "ra_ulysses_all_to_all",
    "ra_ulysses_sim_workspace_bytes", "ra_ulysses_sim_fwd", "ra_usp_sim_workspace_bytes",
    "ra_usp_sim_fwd", "ra_kernel_timing_enable", "ra_kernel_timing_read", "ra_device_info",
    "ra_mfma_probe_bf16", "ra_stream_wait",
)


class RAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class ra_pos(ctypes.Structure):
    _fields_ = [("nseg", ctypes.c_int32), ("seg_len", ctypes.c_int64),
                ("start", ctypes.c_int64 * 2), ("stride", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load (once) and return the library; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RAError(-1, f"HIP library not built: {library_path} is missing "
                          "(run __graft_entry__.build())")
    L = ctypes.CDLL(library_path)
    c_void_p, c_int32, c_int64, c_size_t, c_float = (ctypes.c_void_p, ctypes.c_int32,
                                                      ctypes.c_int64, ctypes.c_size_t,
                                                      ctypes.c_float)
    P = ctypes.POINTER
    sig = {
        "ra_status_str": (ctypes.c_char_p, [c_int32]),
        "ra_last_error": (ctypes.c_char_p, []),
        "ra_block_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int64, c_int32, c_int32]),
        "ra_block_attn_fwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_int32, c_int32, c_int32, c_int64, c_int64, c_int32,
                                        c_int32, P(ra_pos), P(ra_pos), P(c_int32), c_int32,
                                        c_float, c_int32, c_void_p, c_size_t, c_void_p]),
        "ra_block_attn_fwd_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                c_int32, c_int32, c_int32, c_int64, c_int64,
                                                c_int32, c_int32, P(ra_pos), P(ra_pos),
                                                P(c_int32), c_int32, c_float, c_int32, c_void_p]),
        "ra_lse_merge": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                                   c_void_p]),
        "ra_zigzag_permute": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int32,
                                        c_int32, c_void_p]),
        "ra_striped_permute": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int32,
                                         c_int32, c_void_p]),
        "ra_ring_sim_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int64, c_int32,
                                                   c_int32, c_int32]),
        "ra_ring_sim_fwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_int32, c_int32, c_int32, c_int64, c_int32, c_int32,
                                      c_int32, c_int32, c_int32, c_float, P(c_int32),
                                      c_void_p, c_size_t, c_void_p, c_void_p]),
        "ra_block_attn_bwd_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int64,
                                                         c_int64, c_int32, c_int32]),
        "ra_block_attn_bwd": (c_int32, [c_void_p] * 9 + [c_int32, c_int32, c_int32, c_int64,
                                                         c_int64, c_int32, c_int32, P(ra_pos),
                                                         P(ra_pos), P(c_int32), c_int32, c_float,
                                                         c_void_p, c_size_t, c_void_p]),
        "ra_ring_sim_bwd_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int64,
                                                       c_int32, c_int32, c_int32]),
        "ra_ring_sim_bwd": (c_int32, [c_void_p] * 9 + [c_int32, c_int32, c_int32, c_int64,
                                                       c_int32, c_int32, c_int32, c_int32,
                                                       c_int32, c_float, P(c_int32), c_void_p,
                                                       c_size_t, c_void_p]),
        "ra_ulysses_all_to_all": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int32,
                                            c_int64, c_int32, c_int32, c_void_p]),
        "ra_ulysses_sim_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int64,
                                                      c_int32, c_int32, c_int32]),
        "ra_ulysses_sim_fwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_int32, c_int32, c_int32, c_int64, c_int32, c_int32,
                                         c_int32, c_int32, c_float, P(c_int32), c_void_p,
                                         c_size_t, c_void_p]),
        "ra_usp_sim_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int64, c_int32,
                                                  c_int32, c_int32, c_int32]),
        "ra_usp_sim_fwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_int32, c_int32, c_int32, c_int64, c_int32, c_int32,
                                     c_int32, c_int32, c_int32, c_int32, c_float, P(c_int32),
                                     c_void_p, c_size_t, c_void_p, c_void_p]),
        "ra_device_info": (c_int32, [P(c_int32), P(c_int32)]),
        "ra_mfma_probe_bf16": (c_int32, [c_int32, c_void_p, c_int64, P(c_int32), c_void_p]),
        "ra_stream_wait": (c_int32, [c_void_p, c_int32]),
        "ra_kernel_timing_enable": (c_int32, [c_int32]),
        "ra_kernel_timing_read": (c_int32, [P(ctypes.c_double), P(c_int64),
                                            P(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def ra_status_str(status: int) -> str:
    return lib().ra_status_str(status).decode()


def ra_last_error() -> str:
    return lib().ra_last_error().decode()


def _check(status: int):
    if status != 0:
        raise RAError(status, f"{ra_status_str(status)}: {ra_last_error()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    if s is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, torch.cuda.Stream):
        return ctypes.c_void_p(s.cuda_stream)
    return ctypes.c_void_p(int(s))


def _pos(p):
    """None, an ra_pos, or a tuple (nseg, seg_len, start0[, start1[, stride]])."""
    if p is None or isinstance(p, ra_pos):
        return p
    nseg, seg_len, *rest = p
    rest = list(rest) + [0] * (3 - len(rest))
    start0, start1, stride = rest[:3]
    return ra_pos(nseg, seg_len, (ctypes.c_int64 * 2)(start0, start1), stride or 1)


def _kvmap(m, Hq):
    if m is None:
        return None
    m = [int(x) for x in m]
    if len(m) != Hq:
        raise ValueError("kv_head_of_q must have Hq entries")
    return (ctypes.c_int32 * Hq)(*m)


def _dtype(t):
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


# ------------------------------------------------------------------ entry points
def ra_block_attn_workspace_bytes(B, Hkv, Ck, D, dtype) -> int:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().ra_block_attn_workspace_bytes(B, Hkv, Ck, D, dt))


def ra_block_attn_fwd(q, k, v, out, lse, *, q_pos=None, k_pos=None, kv_head_of_q=None,
                      causal=True, scale=None, accumulate=False, workspace=None, stream=None):
    """One block (the pages' flash_block): q [B,Hq,Cq,D], k/v [B,Hkv,Ck,D];
    out fp32 [B,Hq,Cq,D] and lse fp32 [B,Hq,Cq] are the running state."""
    B, Hq, Cq, D = q.shape
    Hkv, Ck = k.shape[1], k.shape[2]
    dt = _dtype(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = ra_block_attn_workspace_bytes(B, Hkv, Ck, D, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    qp, kp = _pos(q_pos), _pos(k_pos)
    _check(lib().ra_block_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Cq, Ck, D, dt,
        ctypes.byref(qp) if qp is not None else None,
        ctypes.byref(kp) if kp is not None else None,
        _kvmap(kv_head_of_q, Hq), int(bool(causal)), float(scale), int(bool(accumulate)),
        _ptr(workspace), wbytes, _stream(stream)))
    return out, lse


def ra_block_attn_fwd_noalloc(q, k, v, out, lse, *, q_pos=None, k_pos=None, kv_head_of_q=None,
                              causal=True, scale=None, accumulate=False, stream=None):
    """ra_block_attn_fwd without a workspace: the transposed V block lives in
    the library's static per-device scratch (see include/ring_attn.h)."""
    B, Hq, Cq, D = q.shape
    Hkv, Ck = k.shape[1], k.shape[2]
    dt = _dtype(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qp, kp = _pos(q_pos), _pos(k_pos)
    _check(lib().ra_block_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Cq, Ck, D, dt,
        ctypes.byref(qp) if qp is not None else None,
        ctypes.byref(kp) if kp is not None else None,
        _kvmap(kv_head_of_q, Hq), int(bool(causal)), float(scale), int(bool(accumulate)),
        _stream(stream)))
    return out, lse


def ra_lse_merge(out, lse, out_b, lse_b, stream=None):
    """In place: (out, lse) <- merge((out, lse), (out_b, lse_b)); out [..., D]."""
    D = out.shape[-1]
    rows = out.numel() // D
    _check(lib().ra_lse_merge(_ptr(out), _ptr(lse), _ptr(out_b), _ptr(lse_b), rows, D,
                              _stream(stream)))
    return out, lse


def ra_zigzag_permute(src, dst, N, inverse=False, seq_dim=-2, stream=None):
    """Zigzag permute along ``seq_dim`` (-2 for [..., S, D], -1 for lse [..., S])."""
    seq_dim = seq_dim % src.dim()
    S = src.shape[seq_dim]
    outer = math.prod(src.shape[:seq_dim])
    row_bytes = math.prod(src.shape[seq_dim + 1:]) * src.element_size()
    _check(lib().ra_zigzag_permute(_ptr(src), _ptr(dst), outer, S, row_bytes, N,
                                   int(bool(inverse)), _stream(stream)))
    return dst


def ra_striped_permute(src, dst, N, inverse=False, seq_dim=-2, stream=None):
    """Striped permute along ``seq_dim`` (-2 for [..., S, D], -1 for lse [..., S])."""
    seq_dim = seq_dim % src.dim()
    S = src.shape[seq_dim]
    outer = math.prod(src.shape[:seq_dim])
    row_bytes = math.prod(src.shape[seq_dim + 1:]) * src.element_size()
    _check(lib().ra_striped_permute(_ptr(src), _ptr(dst), outer, S, row_bytes, N,
                                    int(bool(inverse)), _stream(stream)))
    return dst


_PERMUTES = {"zigzag": ra_zigzag_permute, "striped": ra_striped_permute}


def ra_ring_sim_workspace_bytes(B, Hq, Hkv, S, D, dtype, N) -> int:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().ra_ring_sim_workspace_bytes(B, Hq, Hkv, S, D, dt, N))


def ra_ring_sim_fwd(q, k, v, out, lse, *, N, layout="zigzag", causal=True, scale=None,
                    kv_head_of_q=None, workspace=None, compute_stream=None, copy_stream=None):
    """The simulated N-rank ring on rank-major inputs (see include/ring_attn.h)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dt = _dtype(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(ra_ring_sim_workspace_bytes(B, Hq, Hkv, S, D, dt, N),
                                dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    cs = _stream(compute_stream)
    xs = None if copy_stream is None else _stream(copy_stream)
    _check(lib().ra_ring_sim_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, S, D, dt, N,
        _LAYOUTS[layout] if isinstance(layout, str) else int(layout), int(bool(causal)),
        float(scale), _kvmap(kv_head_of_q, Hq), _ptr(workspace), wbytes, cs, xs))
    return out, lse


def ra_block_attn_bwd_workspace_bytes(B, Hq, Hkv, Cq, Ck, D, dtype) -> int:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().ra_block_attn_bwd_workspace_bytes(B, Hq, Hkv, Cq, Ck, D, dt))


def ra_block_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, *, q_pos=None, k_pos=None,
                      kv_head_of_q=None, causal=True, scale=None, workspace=None, stream=None):
    """Add one block pair's gradients to the fp32 dq, dk, dv (see include/ring_attn.h)."""
    B, Hq, Cq, D = q.shape
    Hkv, Ck = k.shape[1], k.shape[2]
    dt = _dtype(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        n = ra_block_attn_bwd_workspace_bytes(B, Hq, Hkv, Cq, Ck, D, dt)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    qp, kp = _pos(q_pos), _pos(k_pos)
    _check(lib().ra_block_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
        _ptr(dv), B, Hq, Hkv, Cq, Ck, D, dt,
        None if qp is None else ctypes.byref(qp), None if kp is None else ctypes.byref(kp),
        _kvmap(kv_head_of_q, Hq), int(bool(causal)), float(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def ra_ring_sim_bwd_workspace_bytes(B, Hq, Hkv, S, D, dtype, N) -> int:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().ra_ring_sim_bwd_workspace_bytes(B, Hq, Hkv, S, D, dt, N))


def ra_ring_sim_bwd(q, k, v, out, dout, lse, dq, dk, dv, *, N, layout="zigzag", causal=True,
                    scale=None, kv_head_of_q=None, workspace=None, stream=None):
    """The simulated N-rank ring backward on rank-major tensors (see include/ring_attn.h)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dt = _dtype(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(max(ra_ring_sim_bwd_workspace_bytes(B, Hq, Hkv, S, D, dt, N), 1),
                                dtype=torch.uint8, device=q.device)
    _check(lib().ra_ring_sim_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
        _ptr(dv), B, Hq, Hkv, S, D, dt, N,
        _LAYOUTS[layout] if isinstance(layout, str) else int(layout), int(bool(causal)),
        float(scale), _kvmap(kv_head_of_q, Hq), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def ra_ulysses_all_to_all(src, dst, P, inverse=False, stream=None):
    """Ulysses all-to-all of P ranks (see include/ring_attn.h). Forward: src
    [P, B, S/P, H, row...] -> dst [P, B, H/P, S, row...]; inverse the reverse."""
    if not inverse:
        _, B, Sp, H = src.shape[:4]
        S = Sp * P
        row = src.shape[4:]
    else:
        _, B, Hp, S = src.shape[:4]
        H = Hp * P
        row = src.shape[4:]
    row_bytes = math.prod(row) * src.element_size()
    _check(lib().ra_ulysses_all_to_all(_ptr(src), _ptr(dst), B, S, H, row_bytes, P,
                                       int(bool(inverse)), _stream(stream)))
    return dst


def ra_ulysses_sim_workspace_bytes(B, Hq, Hkv, S, D, dtype, P) -> int:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().ra_ulysses_sim_workspace_bytes(B, Hq, Hkv, S, D, dt, P))


def ra_ulysses_sim_fwd(q, k, v, out, lse, *, P, causal=True, scale=None, kv_head_of_q=None,
                       workspace=None, stream=None):
    """Ulysses attention of P ranks on one GPU. q, out: [P, B, S/P, Hq, D];
    k, v: [P, B, S/P, Hkv, D]; lse: float32 [P, B, Hq/P, S]."""
    _, B, Sp, Hq, D = q.shape
    Hkv = k.shape[3]
    S = Sp * P
    dt = _dtype(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(ra_ulysses_sim_workspace_bytes(B, Hq, Hkv, S, D, dt, P),
                                dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().ra_ulysses_sim_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, S, D, dt, P,
        int(bool(causal)), float(scale), _kvmap(kv_head_of_q, Hq), _ptr(workspace), wbytes,
        _stream(stream)))
    return out, lse


def ra_usp_sim_workspace_bytes(B, Hq, Hkv, S, D, dtype, P_u, P_r) -> int:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().ra_usp_sim_workspace_bytes(B, Hq, Hkv, S, D, dt, P_u, P_r))


def ra_usp_sim_fwd(q, k, v, out, lse, *, P_u, P_r, layout="zigzag", causal=True, scale=None,
                   kv_head_of_q=None, workspace=None, compute_stream=None, copy_stream=None):
    """USP on a P_r x P_u grid on one GPU. q, out: [P_r*P_u, B, S/(P_r*P_u), Hq, D];
    k, v: [.., Hkv, D]; lse: float32 [P_u, B, Hq/P_u, S] (see include/ring_attn.h)."""
    _, B, Sp, Hq, D = q.shape
    Hkv = k.shape[3]
    S = Sp * P_u * P_r
    dt = _dtype(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(ra_usp_sim_workspace_bytes(B, Hq, Hkv, S, D, dt, P_u, P_r),
                                dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    xs = None if copy_stream is None else _stream(copy_stream)
    _check(lib().ra_usp_sim_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, S, D, dt, P_u, P_r,
        _LAYOUTS[layout] if isinstance(layout, str) else int(layout), int(bool(causal)),
        float(scale), _kvmap(kv_head_of_q, Hq), _ptr(workspace), wbytes,
        _stream(compute_stream), xs))
    return out, lse


def ra_device_info():
    """(compute units, maximum shader clock in kHz) of the current device."""
    cus, khz = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ra_device_info(ctypes.byref(cus), ctypes.byref(khz)))
    return cus.value, khz.value


def ra_stream_wait(stream=None, timeout_ms=60000):
    """Wait until everything enqueued on `stream` so far has run, for at most
    timeout_ms milliseconds; raises RAError with status RA_ERR_TIMEOUT when
    the stream is still busy then (its work is left running)."""
    _check(lib().ra_stream_wait(_stream(stream), int(timeout_ms)))


def ra_mfma_probe_bf16(iters=100000, device=None):
    """Run the matrix-core probe once (after a short warm-up launch) and
    return its figures: dense bf16 flops per compute unit per clock and the
    shader clock (median over workgroups, each over its own span from the
    earliest start to the latest end of its 8 waves), and the chip rate over
    the whole launch (HIP events)."""
    dev = torch.device(device) if device is not None else torch.device("cuda",
                                                                       torch.cuda.current_device())
    cus, _ = ra_device_info()
    words = 5
    buf = torch.zeros(words * 8 * cus, dtype=torch.int64, device=dev)
    waves = ctypes.c_int32()
    stream = _stream(None)
    _check(lib().ra_mfma_probe_bf16(max(1, iters // 10), _ptr(buf), buf.numel(),
                                    ctypes.byref(waves), stream))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    _check(lib().ra_mfma_probe_bf16(iters, _ptr(buf), buf.numel(), ctypes.byref(waves), stream))
    e1.record()
    torch.cuda.synchronize()
    rec = buf.view(-1, 8, words)[:waves.value // 8].cpu()
    cycles = (rec[:, :, 1].max(dim=1).values - rec[:, :, 0].min(dim=1).values).double()
    ticks = (rec[:, :, 3].max(dim=1).values - rec[:, :, 2].min(dim=1).values).double()
    flops_wg = 8 * 4 * iters * 32768.0
    ms = e0.elapsed_time(e1)
    return {"flops_per_cu_clk": (flops_wg / cycles).median().item(),
            "clock_mhz": (cycles / (ticks / 100.0)).median().item(),
            "chip_tflops": flops_wg * (waves.value // 8) / (ms * 1e-3) / 1e12,
            "waves": waves.value, "iters": iters}


def ra_kernel_timing_enable(enable=True):
    _check(lib().ra_kernel_timing_enable(int(bool(enable))))


def ra_kernel_timing_read():
    """Returns (total_ms, launches, useful_flops) and clears the record."""
    ms, n, fl = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double()
    _check(lib().ra_kernel_timing_read(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl)))
    return ms.value, n.value, fl.value


# ------------------------------------------------------------------ convenience
class RingRunner:
    """Owns the buffers of repeated ring calls on one shape (allocated once)."""

    def __init__(self, B, Hq, Hkv, S, D, dtype, N, layout="zigzag", causal=True, scale=None,
                 kv_head_of_q=None, device="cuda", copy_stream=True):
        self.shape = (B, Hq, Hkv, S, D)
        self.N, self.layout, self.causal = N, layout, causal
        self.scale = 1.0 / math.sqrt(D) if scale is None else scale
        self.kv_head_of_q = kv_head_of_q
        self.dtype = dtype
        dev = torch.device(device)
        self.workspace = torch.empty(ra_ring_sim_workspace_bytes(B, Hq, Hkv, S, D, dtype, N),
                                     dtype=torch.uint8, device=dev)
        self.out_rm = torch.empty((B, Hq, S, D), dtype=dtype, device=dev)
        self.lse_rm = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        self.copy_stream = torch.cuda.Stream(device=dev) if copy_stream else None
        if layout in _PERMUTES:
            self.q_rm = torch.empty((B, Hq, S, D), dtype=dtype, device=dev)
            self.k_rm = torch.empty((B, Hkv, S, D), dtype=dtype, device=dev)
            self.v_rm = torch.empty((B, Hkv, S, D), dtype=dtype, device=dev)

    def permute_inputs(self, q, k, v):
        perm = _PERMUTES.get(self.layout)
        if perm is None:
            return q, k, v
        perm(q, self.q_rm, self.N)
        perm(k, self.k_rm, self.N)
        perm(v, self.v_rm, self.N)
        return self.q_rm, self.k_rm, self.v_rm

    def ring(self, q_rm, k_rm, v_rm):
        return ra_ring_sim_fwd(q_rm, k_rm, v_rm, self.out_rm, self.lse_rm, N=self.N,
                               layout=self.layout, causal=self.causal, scale=self.scale,
                               kv_head_of_q=self.kv_head_of_q, workspace=self.workspace,
                               copy_stream=self.copy_stream)

    def unpermute_outputs(self, out, lse):
        perm = _PERMUTES.get(self.layout)
        if perm is None:
            out.copy_(self.out_rm)
            lse.copy_(self.lse_rm)
            return out, lse
        perm(self.out_rm, out, self.N, inverse=True)
        perm(self.lse_rm, lse, self.N, inverse=True, seq_dim=-1)
        return out, lse

    def __call__(self, q, k, v, out, lse):
        """Whole step in sequence order: permute, ring, inverse permute."""
        self.ring(*self.permute_inputs(q, k, v))
        return self.unpermute_outputs(out, lse)


def ring_attention_sim_backward(q, k, v, out, lse, dout, *, N, layout="zigzag", causal=True,
                                scale=None, kv_head_of_q=None, workspace=None):
    """Sequence-order tensors in (out, lse from the forward), sequence-order (dq, dk, dv) out."""
    perm = _PERMUTES.get(layout)

    def fwd(t, seq_dim=-2):
        if perm is None:
            return t
        dst = torch.empty_like(t)
        perm(t, dst, N, seq_dim=seq_dim)
        return dst

    def inv(t):
        if perm is None:
            return t
        dst = torch.empty_like(t)
        perm(t, dst, N, inverse=True)
        return dst

    qr, kr, vr, outr, doutr = (fwd(t) for t in (q, k, v, out, dout))
    lser = fwd(lse, seq_dim=-1)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ra_ring_sim_bwd(qr, kr, vr, outr, doutr, lser, dq, dk, dv, N=N, layout=layout,
                    causal=causal, scale=scale, kv_head_of_q=kv_head_of_q, workspace=workspace)
    return inv(dq), inv(dk), inv(dv)


def ring_attention_sim(q, k, v, *, N, layout="zigzag", causal=True, scale=None,
                       kv_head_of_q=None):
    """Sequence-order inputs in, sequence-order (out, lse) out."""
    B, Hq, S, D = q.shape
    r = RingRunner(B, Hq, k.shape[1], S, D, q.dtype, N, layout, causal, scale, kv_head_of_q,
                   device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    return r(q, k, v, out, lse)
