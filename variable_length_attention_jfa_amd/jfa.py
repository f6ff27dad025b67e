"""Python binding of libjfa.so (ctypes): argument marshalling only.

Every step of the computation runs in the library's gfx950 kernels. PyTorch
provides device memory and the current HIP stream; nothing here computes
attention, and there is no fallback: if the library is not built or the device
is not an MI355X, calls raise.

    out, lse = forward(q, k, v, q_offsets, kv_offsets, bias=None, causal=False, max_kv_len=0)
    dq, dk, dv = backward(q, k, v, out, lse, dout, q_offsets, kv_offsets, bias, causal, max_kv_len=0)

Tensors: q/out/dout [Tq, H, D], k/v [Tk, H, D] (bf16 or fp32, contiguous, on
the GPU); offsets int32 [B+1] on the GPU; bias fp32 [H, 257] or None; lse fp32
[Tq, H] (natural log).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjfa.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "jfa.h")

KERNEL_FWD, KERNEL_BWD_DKDV, KERNEL_BWD_DQ, KERNEL_BWD_SQ, KERNEL_FWD_SQ = 0, 1, 2, 3, 4
SQ_KERNELS = (KERNEL_BWD_SQ, KERNEL_FWD_SQ)  # short-query chunk lists (one list, two passes)
DTYPE_BF16, DTYPE_F32 = 0, 1
BIAS_RADIUS = 128
ABI_VERSION = 5  # JFA_ABI_VERSION of include/jfa.h
WORKSPACE_ALIGN = 256
PLAN_HEADER_BYTES = 2048
PLAN_QUEUES = 8

_LIB = None

_vp, _i32p, _f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_int, _i64, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t

_SIGS = {
    "jfa_abi_version": (_int, []),
    "jfa_fwd_workspace_bytes": (_sz, [_int, _int, _i64, _i64, _int, _int]),
    "jfa_bwd_workspace_bytes": (_sz, [_int, _int, _i64, _i64, _int, _int]),
    "jfa_fwd": (_int, [_vp, _vp, _vp, _i32p, _i32p, _int, _int, _int, _i64, _i64, _int, _f32p, _int, _vp, _f32p, _vp, _sz,
                       _vp]),
    "jfa_fwd_noalloc": (_int, [_vp, _vp, _vp, _i32p, _i32p, _int, _int, _int, _i64, _i64, _int, _f32p, _int, _vp, _f32p,
                               _vp]),
    "jfa_fwd_f32": (_int, [_vp, _vp, _vp, _i32p, _i32p, _int, _int, _int, _i64, _i64, _int, _f32p, _int, _vp, _f32p, _vp,
                           _sz, _vp]),
    "jfa_bwd": (_int, [_vp, _vp, _vp, _vp, _f32p, _vp, _i32p, _i32p, _int, _int, _int, _i64, _i64, _int, _f32p, _int,
                       _vp, _vp, _vp, _f32p, _vp, _sz, _vp]),
    "jfa_bwd_f32": (_int, [_vp, _vp, _vp, _vp, _f32p, _vp, _i32p, _i32p, _int, _int, _int, _i64, _i64, _int, _f32p, _int,
                           _vp, _vp, _vp, _f32p, _vp, _sz, _vp]),
    "jfa_padded_workspace_bytes": (_sz, [_int, _int, _int, _int, _int]),
    "jfa_fwd_padded": (_int, [_vp, _vp, _vp, _i32p, _int, _int, _int, _int, _int, _f32p, _int, _vp, _f32p, _vp, _sz, _vp]),
    "jfa_bwd_padded": (_int, [_vp, _vp, _vp, _vp, _f32p, _vp, _i32p, _int, _int, _int, _int, _int, _f32p, _int, _vp,
                              _vp, _vp, _vp, _sz, _vp]),
    "jfa_offsets_from_lengths": (_int, [_i32p, _int, _i32p, _vp]),
    "jfa_tile_config": (_int, [_int, _int, _int, ctypes.POINTER(_int), ctypes.POINTER(_int)]),
    "jfa_build_plan": (_int, [_i32p, _i32p, _int, _int, _int, _int, _int, _int, _vp, _sz, _vp]),
    "jfa_plan_workspace_bytes": (_sz, [_int, _int, _i64, _i64, _int, _int, _int]),
    "jfa_timing_enable": (_int, [_int]),
    "jfa_timing_collect": (_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), _int]),
    "jfa_status_string": (ctypes.c_char_p, [_int]),
    "jfa_last_error": (ctypes.c_char_p, []),
}


class JFAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m variable_length_attention_jfa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        # argument lists must match the ones below: a library built from
        # older sources would read the arguments wrongly
        ver = getattr(L, "jfa_abi_version", None)
        if ver is None or ver() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} was built for another ABI version (rebuild it)")
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def declared_functions() -> list:
    """Names of the functions include/jfa.h declares."""
    with open(HEADER_PATH) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jfa_\w+)\s*\(", text)))


def _check(fn: str, status: int) -> None:
    if status != 0:
        L = lib()
        raise JFAError(fn, status, f"{L.jfa_status_string(status).decode()}: {L.jfa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(nbytes: int, device) -> Tuple[torch.Tensor, int]:
    buf = torch.empty(nbytes + WORKSPACE_ALIGN, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % WORKSPACE_ALIGN
    return buf, buf.data_ptr() + off


def _check_tensor(name: str, t: torch.Tensor, dtype, dims: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.dim() != dims or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dims}-d tensor")


def _check_shape(name: str, t: torch.Tensor, shape) -> None:
    # the library writes through plain pointers: a buffer smaller than its
    # tensor's logical size would be written past its end
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _common(q, k, v, q_offsets, kv_offsets, bias):
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q/k/v must be bfloat16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.dtype, 3)
    _check_tensor("q_offsets", q_offsets, torch.int32, 1)
    _check_tensor("kv_offsets", kv_offsets, torch.int32, 1)
    Tq, H, D = q.shape
    Tk = k.shape[0]
    if k.shape[1:] != (H, D) or v.shape != k.shape:
        raise ValueError("k and v must be [Tk, H, D] with q's H and D")
    B = q_offsets.numel() - 1
    if kv_offsets.numel() != B + 1 or B < 0:
        raise ValueError("q_offsets and kv_offsets must both have B+1 entries")
    if bias is not None:
        _check_tensor("bias", bias, torch.float32, 2)
        if bias.shape != (H, 2 * BIAS_RADIUS + 1):
            raise ValueError(f"bias must be [H, {2 * BIAS_RADIUS + 1}]")
    return B, H, D, Tq, Tk


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_offsets: torch.Tensor, kv_offsets: torch.Tensor,
            bias: Optional[torch.Tensor] = None, causal: bool = False, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, max_kv_len: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """max_kv_len: an upper bound on every sequence's key count if known on the host, else 0 (a bound of at
    most 1024 skips the short-query launches; a wrong bound costs speed only)."""
    B, H, D, Tq, Tk = _common(q, k, v, q_offsets, kv_offsets, bias)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=q.device)
    _check_tensor("out", out, q.dtype, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    _check_shape("out", out, q.shape)
    _check_shape("lse", lse, (Tq, H))
    L = lib()
    nbytes = L.jfa_fwd_workspace_bytes(B, H, Tq, Tk, D, int(causal))
    ws, wp = _workspace(nbytes, q.device)
    fn = L.jfa_fwd_f32 if q.dtype == torch.float32 else L.jfa_fwd
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets), B, H, D, Tq, Tk, int(max_kv_len), _ptr(bias),
            int(causal), _ptr(out), _ptr(lse), ctypes.c_void_p(wp), nbytes, _stream())
    _check("jfa_fwd", st)
    return out, lse


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_offsets: torch.Tensor,
                    kv_offsets: torch.Tensor, bias: Optional[torch.Tensor], causal: bool, out: torch.Tensor,
                    lse: torch.Tensor, max_kv_len: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """jfa_fwd_noalloc: the forward with the library's fixed scratch instead of a
    workspace (bf16; out and lse are the caller's, nothing is allocated)."""
    B, H, D, Tq, Tk = _common(q, k, v, q_offsets, kv_offsets, bias)
    if q.dtype != torch.bfloat16:
        raise ValueError("jfa_fwd_noalloc takes bfloat16 tensors")
    _check_tensor("out", out, q.dtype, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    _check_shape("out", out, q.shape)
    _check_shape("lse", lse, (Tq, H))
    st = lib().jfa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets), B, H, D, Tq, Tk,
                               int(max_kv_len), _ptr(bias), int(causal), _ptr(out), _ptr(lse), _stream())
    _check("jfa_fwd_noalloc", st)
    return out, lse


def backward(q, k, v, out, lse, dout, q_offsets, kv_offsets, bias=None, causal: bool = False,
             dq=None, dk=None, dv=None, bias_grad: bool = False, max_kv_len: int = 0):
    """Gradients (dq, dk, dv); with bias_grad also the fp32 [H, 257] gradient of the bias table.
    max_kv_len: as for forward."""
    B, H, D, Tq, Tk = _common(q, k, v, q_offsets, kv_offsets, bias)
    if bias_grad and bias is None:
        raise ValueError("bias_grad needs a bias")
    _check_tensor("out", out, q.dtype, 3)
    _check_tensor("dout", dout, q.dtype, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, q.dtype, 3)
        _check_shape(name, t, ref.shape)
    _check_shape("lse", lse, (Tq, H))
    L = lib()
    nbytes = L.jfa_bwd_workspace_bytes(B, H, Tq, Tk, D, int(causal))
    ws, wp = _workspace(nbytes, q.device)
    fn = L.jfa_bwd_f32 if q.dtype == torch.float32 else L.jfa_bwd
    dbias = torch.empty((H, 2 * BIAS_RADIUS + 1), dtype=torch.float32, device=q.device) if bias_grad else None
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(q_offsets), _ptr(kv_offsets), B, H, D,
            Tq, Tk, int(max_kv_len), _ptr(bias), int(causal), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
            ctypes.c_void_p(wp), nbytes, _stream())
    _check("jfa_bwd", st)
    return (dq, dk, dv, dbias) if bias_grad else (dq, dk, dv)


def _padded_common(q, k, v, bias):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16, 4)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape[0] != B or k.shape[2:] != (H, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, kv_slot, H, D] with q's B, H and D")
    if bias is not None:
        _check_tensor("bias", bias, torch.float32, 2)
        if bias.shape != (H, 2 * BIAS_RADIUS + 1):
            raise ValueError(f"bias must be [H, {2 * BIAS_RADIUS + 1}]")
    return B, Sq, Sk, H, D


def forward_padded(q, k, v, kv_lens, bias=None, causal: bool = False, out=None, lse=None):
    """Padded-dense baseline forward: q [B, q_slot, H, D], k/v [B, kv_slot, H, D] bf16, kv_lens int32 [B] on
    the GPU (true key counts). Returns (out [B, q_slot, H, D], lse fp32 [B, q_slot, H]); rows past a
    sequence's true query length are not meaningful."""
    B, Sq, Sk, H, D = _padded_common(q, k, v, bias)
    _check_tensor("kv_lens", kv_lens, torch.int32, 1)
    if kv_lens.numel() != B:
        raise ValueError("kv_lens must have B entries")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, q.dtype, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    _check_shape("out", out, q.shape)
    _check_shape("lse", lse, (B, Sq, H))
    L = lib()
    nbytes = L.jfa_padded_workspace_bytes(B, H, Sq, Sk, D)
    if nbytes == 0:
        raise ValueError("invalid padded sizes")
    ws, wp = _workspace(nbytes, q.device)
    st = L.jfa_fwd_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_lens), B, Sq, Sk, H, D, _ptr(bias), int(causal),
                          _ptr(out), _ptr(lse), ctypes.c_void_p(wp), nbytes, _stream())
    _check("jfa_fwd_padded", st)
    return out, lse


def backward_padded(q, k, v, out, lse, dout, kv_lens, bias=None, causal: bool = False, dq=None, dk=None, dv=None):
    """Padded-dense baseline backward (pad rows of q, k, v, dout must be zero); returns (dq, dk, dv)."""
    B, Sq, Sk, H, D = _padded_common(q, k, v, bias)
    _check_tensor("kv_lens", kv_lens, torch.int32, 1)
    if kv_lens.numel() != B:
        raise ValueError("kv_lens must have B entries")
    _check_tensor("lse", lse, torch.float32, 3)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, t, q.dtype, 4)
        _check_shape(name, t, ref.shape)
    _check_shape("lse", lse, (B, Sq, H))
    L = lib()
    nbytes = L.jfa_padded_workspace_bytes(B, H, Sq, Sk, D)
    if nbytes == 0:
        raise ValueError("invalid padded sizes")
    ws, wp = _workspace(nbytes, q.device)
    st = L.jfa_bwd_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(kv_lens), B, Sq, Sk, H, D,
                          _ptr(bias),
                          int(causal), _ptr(dq), _ptr(dk), _ptr(dv), ctypes.c_void_p(wp), nbytes, _stream())
    _check("jfa_bwd_padded", st)
    return dq, dk, dv


def offsets_from_lengths(lengths: torch.Tensor) -> torch.Tensor:
    _check_tensor("lengths", lengths, torch.int32, 1)
    B = lengths.numel()
    offsets = torch.empty(B + 1, dtype=torch.int32, device=lengths.device)
    _check("jfa_offsets_from_lengths", lib().jfa_offsets_from_lengths(_ptr(lengths), B, _ptr(offsets), _stream()))
    return offsets


def tile_config(kernel: int, D: int, dtype: int = DTYPE_BF16) -> Tuple[int, int]:
    tm, tn = _int(0), _int(0)
    _check("jfa_tile_config", lib().jfa_tile_config(kernel, D, dtype, ctypes.byref(tm), ctypes.byref(tn)))
    return tm.value, tn.value


def build_plan(q_offsets: torch.Tensor, kv_offsets: torch.Tensor, H: int, D: int, causal: bool, kernel: int,
               total_q: int, total_kv: int, dtype: int = DTYPE_BF16) -> Tuple[torch.Tensor, torch.Tensor]:
    """Runs the on-device work-list builder; returns (header int32[512], items int32[n, 4]) on the device,
    and for the short-query lists (KERNEL_BWD_SQ, KERNEL_FWD_SQ) also the per-(b, h) position of chunk 0
    (int32[B*H], -1 if none)."""
    _check_tensor("q_offsets", q_offsets, torch.int32, 1)
    _check_tensor("kv_offsets", kv_offsets, torch.int32, 1)
    B = q_offsets.numel() - 1
    L = lib()
    nbytes = L.jfa_plan_workspace_bytes(B, H, total_q, total_kv, D, dtype, kernel)
    if nbytes == 0:
        raise ValueError("invalid plan sizes")
    ws, wp = _workspace(nbytes, q_offsets.device)
    st = L.jfa_build_plan(_ptr(q_offsets), _ptr(kv_offsets), B, H, D, dtype, int(causal), kernel, ctypes.c_void_p(wp),
                          nbytes, _stream())
    _check("jfa_build_plan", st)
    off = wp - ws.data_ptr()
    tail = (B * H * 4 + 255) // 256 * 256 if kernel in SQ_KERNELS else 0
    header = ws[off:off + PLAN_HEADER_BYTES].view(torch.int32)
    items = ws[off + PLAN_HEADER_BYTES:off + nbytes - tail].view(torch.int32).view(-1, 4)
    if kernel not in SQ_KERNELS:
        return header, items
    return header, items, ws[off + nbytes - tail:off + nbytes - tail + B * H * 4].view(torch.int32)


TIMING_KINDS = ("plan", "forward", "bwd_prep", "dkdv", "dq", "scan", "sq", "fsq", "dbias")


def timing_enable(enable: bool = True) -> None:
    _check("jfa_timing_enable", lib().jfa_timing_enable(int(enable)))


def timing_collect() -> dict:
    """{kind: (total_ms, launches)} for launches since the last collect."""
    n = len(TIMING_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check("jfa_timing_collect", lib().jfa_timing_collect(ms, cnt, n))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(TIMING_KINDS)}


class JaggedAttention(torch.autograd.Function):
    """autograd wrapper: O = jagged attention(q, k, v); gradients via jfa_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, q_offsets, kv_offsets, bias=None, causal=False, max_kv_len=0):
        out, lse = forward(q, k, v, q_offsets, kv_offsets, bias, causal, max_kv_len=max_kv_len)
        ctx.save_for_backward(q, k, v, out, lse, q_offsets, kv_offsets, bias)
        ctx.causal = causal
        ctx.max_kv_len = max_kv_len
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, qo, ko, bias = ctx.saved_tensors
        want_db = bias is not None and ctx.needs_input_grad[5]
        g = backward(q, k, v, out, lse, dout.contiguous(), qo, ko, bias, ctx.causal, bias_grad=want_db,
                     max_kv_len=ctx.max_kv_len)
        return g[0], g[1], g[2], None, None, (g[3] if want_db else None), None, None


def jagged_attention(q, k, v, q_offsets, kv_offsets, bias=None, causal=False, max_kv_len=0):
    return JaggedAttention.apply(q, k, v, q_offsets, kv_offsets, bias, causal, max_kv_len)
