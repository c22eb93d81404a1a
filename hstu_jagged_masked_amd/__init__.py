"""HSTU jagged masked attention on MI355X (gfx950): Python binding.

A thin ctypes layer over ``libhstu_attn.so`` (built in-tree by
``hstu_jagged_masked_amd.build``).  It only marshals arguments: every step of
the operator runs in the library's HIP kernels.  PyTorch provides device
memory and the current stream.  There is no CPU or PyTorch fallback: if the
library is missing the import of the op raises.

Entry points mirror the C ABI (include/hstu_attn.h):

    attn_fwd(q, k, v, seq_offsets, func, alpha, max_len, target_rows=None) -> o
    attn_fwd_noalloc(...)  # the same without a workspace (fixed per-device array)
    attn_bwd(q, k, v, dout, seq_offsets, func, alpha, max_len, target_rows=None,
             pstore=None) -> dq, dk, dv
    pstore_bytes(seq_offsets, H) -> bytes of the stored-P buffer attn_bwd(pstore=...) needs
    visible_counts(seq_offsets, func, total, target_rows=None) -> (counts, total_pairs)
    check_inputs(seq_offsets, total, target_rows=None)
    hstu_attention(...)  # autograd.Function wrapper of the two above

Tensors: q, k, v, dout are CUDA tensors ``[rows, H, D]`` (bfloat16 or float32,
contiguous); in targets-only mode q and dout are ``[B, H, D]``.  ``seq_offsets``
is int64 ``[B+1]``, ``func`` int32 ``[nfunc, total]``, ``target_rows`` int32
``[B]``, all on the same device.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libhstu_attn.so")

HSTU_BF16 = 0
HSTU_FP32 = 1
_STATUS = {0: "OK", -1: "invalid argument", -2: "unsupported", -3: "workspace too small",
           -4: "device error", -5: "malformed input"}

_lib = None


class HstuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hstu_attn: {_STATUS.get(status, status)}: {message}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load libhstu_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is missing: build it with "
                          "`python -m hstu_jagged_masked_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIBRARY)
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.hstu_max_nfunc.argtypes = []
    lib.hstu_max_nfunc.restype = i32
    lib.hstu_last_error.argtypes = []
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_attn_workspace_size.argtypes = [i32, i64, i64, i32, i32, i32, i32]
    lib.hstu_attn_workspace_size.restype = sz
    lib.hstu_attn_fwd.argtypes = [i32, P, P, P, P, P, i64, i64, i32, i32, P, i32, f32, i64, P, P,
                                  sz, P]
    lib.hstu_attn_fwd.restype = i32
    lib.hstu_attn_fwd_noalloc.argtypes = [i32, P, P, P, P, P, i64, i64, i32, i32, P, i32, f32,
                                          i64, P, P]
    lib.hstu_attn_fwd_noalloc.restype = i32
    lib.hstu_attn_bwd.argtypes = [i32, P, P, P, P, P, P, P, P, i64, i64, i32, i32, P, i32, f32,
                                  i64, P, P, sz, P]
    lib.hstu_attn_bwd.restype = i32
    lib.hstu_attn_visible_counts.argtypes = [P, i64, i64, P, i32, P, P, P, P]
    lib.hstu_attn_visible_counts.restype = i32
    lib.hstu_attn_check_inputs.argtypes = [P, i64, i64, P, P, sz, P]
    lib.hstu_attn_check_inputs.restype = i32
    lib.hstu_attn_bwd_pstore.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i32, i32, P, i32, f32,
                                         i64, P, sz, P, sz, P]
    lib.hstu_attn_bwd_pstore.restype = i32
    lib.hstu_attn_bwd_pstore_chunked.argtypes = [P, P, P, P, P, P, P, P, P, i64, i64, i32, i32, P,
                                                 i32, f32, i64, P, sz, P, sz, P]
    lib.hstu_attn_bwd_pstore_chunked.restype = i32
    lib.hstu_attn_bwd_atomic.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i32, i32, P, i32, f32,
                                         i64, P, sz, P, sz, P]
    lib.hstu_attn_bwd_atomic.restype = i32
    lib.hstu_attn_pstore_bytes.argtypes = [P, i64, i64, i32]
    lib.hstu_attn_pstore_bytes.restype = sz
    lib.hstu_profile_enable.argtypes = [i32]
    lib.hstu_profile_enable.restype = i32
    lib.hstu_profile_read.argtypes = [ctypes.c_char_p, sz]
    lib.hstu_profile_read.restype = sz
    lib.hstu_profile_reset.argtypes = []
    lib.hstu_profile_reset.restype = None
    _lib = lib
    return lib


EXPORTED = ("hstu_max_nfunc", "hstu_last_error", "hstu_attn_workspace_size", "hstu_attn_fwd",
            "hstu_attn_fwd_noalloc", "hstu_attn_bwd", "hstu_attn_bwd_pstore", "hstu_attn_bwd_pstore_chunked",
            "hstu_attn_bwd_atomic",
            "hstu_attn_pstore_bytes",
            "hstu_attn_visible_counts", "hstu_attn_check_inputs",
            "hstu_profile_enable", "hstu_profile_read", "hstu_profile_reset")


def _check(status: int):
    if status != 0:
        msg = library().hstu_last_error()
        raise HstuError(status, msg.decode() if msg else "")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HSTU_BF16
    if t.dtype == torch.float32:
        return HSTU_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def max_nfunc() -> int:
    return library().hstu_max_nfunc()


def workspace_size(is_bwd, B, total, H, D, nfunc, targets_only) -> int:
    return int(library().hstu_attn_workspace_size(int(is_bwd), int(B), int(total), int(H), int(D),
                                                  int(nfunc), int(targets_only)))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _common(q, k, seq_offsets, func, target_rows):
    if k.dim() != 3:
        raise ValueError("k must be [total, H, D]")
    total, H, D = k.shape
    B = seq_offsets.numel() - 1
    if func.dim() != 2 or func.shape[1] != total:
        raise ValueError("func must be [nfunc, total] int32")
    if seq_offsets.dtype != torch.int64 or func.dtype != torch.int32:
        raise TypeError("seq_offsets must be int64 and func int32")
    if target_rows is not None:
        if target_rows.dtype != torch.int32 or target_rows.numel() != B:
            raise ValueError("target_rows must be int32 [B]")
        if q.shape[0] != B:
            raise ValueError("in targets-only mode q must be [B, H, D]")
    elif q.shape[0] != total:
        raise ValueError("q must be [total, H, D]")
    for t in (seq_offsets, func, target_rows):
        if t is not None and not t.is_contiguous():
            raise ValueError("seq_offsets, func and target_rows must be contiguous")
    return B, total, H, D, func.shape[0]


def attn_fwd(q, k, v, seq_offsets, func, alpha, max_len, target_rows=None, out=None):
    B, total, H, D, nfunc = _common(q, k, seq_offsets, func, target_rows)
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != k.dtype:
            raise ValueError("q, k, v must be contiguous and share a dtype")
    code = _dtype_code(k)
    o = torch.empty_like(q) if out is None else out
    ws_bytes = workspace_size(0, B, total, H, D, nfunc, target_rows is not None)
    ws = _workspace(ws_bytes, k.device)
    _check(library().hstu_attn_fwd(
        code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_offsets), B, total, H, D, _ptr(func),
        nfunc, float(alpha), int(max_len), _ptr(target_rows), _ptr(ws), ws.numel(),
        _stream(k.device)))
    return o


def attn_fwd_noalloc(q, k, v, seq_offsets, func, alpha, max_len, target_rows=None, out=None):
    """attn_fwd through the entry point that takes no workspace (the library's
    fixed per-device array serves instead; larger sizes raise).  ``out`` lets a
    caller that cannot allocate pass the output buffer too."""
    B, total, H, D, nfunc = _common(q, k, seq_offsets, func, target_rows)
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != k.dtype:
            raise ValueError("q, k, v must be contiguous and share a dtype")
    code = _dtype_code(k)
    o = torch.empty_like(q) if out is None else out
    _check(library().hstu_attn_fwd_noalloc(
        code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_offsets), B, total, H, D, _ptr(func),
        nfunc, float(alpha), int(max_len), _ptr(target_rows), _stream(k.device)))
    return o


def pstore_bytes(seq_offsets, H) -> int:
    """Bytes of the stored-P buffer for attn_bwd(pstore=...): the sum over
    sequences of ceil(L/128) * ceil(L/32) * 8192 * H (reads the offsets back
    to the host)."""
    off = seq_offsets.detach().to("cpu", torch.int64).contiguous()
    B = off.numel() - 1
    total = int(off[-1].item()) if B >= 0 else 0
    return int(library().hstu_attn_pstore_bytes(ctypes.c_void_p(off.data_ptr()), B, total, int(H)))


def attn_bwd(q, k, v, dout, seq_offsets, func, alpha, max_len, target_rows=None, pstore=None,
             host_offsets=None):
    """Backward.  With ``pstore`` (a CUDA uint8 tensor of at least
    ``pstore_bytes(seq_offsets, H)`` bytes; bf16, D = 128, full-length mode) the
    stored-P path runs: no recomputation of the scores for dQ.  The size is
    checked on the device: with a smaller buffer dq comes back as NaN.
    With ``host_offsets`` as well (a CPU int64 copy of seq_offsets), ``pstore``
    may be of any size that holds the largest sequence's P: the batch runs in
    runs of sequences that fit it, with the same outputs."""
    B, total, H, D, nfunc = _common(q, k, seq_offsets, func, target_rows)
    for t in (q, k, v, dout):
        if not t.is_contiguous() or t.dtype != k.dtype:
            raise ValueError("q, k, v, dout must be contiguous and share a dtype")
    code = _dtype_code(k)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws_bytes = workspace_size(1, B, total, H, D, nfunc, target_rows is not None)
    ws = _workspace(ws_bytes, k.device)
    if pstore is not None:
        if target_rows is not None or code != HSTU_BF16:
            raise ValueError("the stored-P backward needs bf16 and full-length mode")
        if pstore.dtype != torch.uint8 or not pstore.is_contiguous():
            raise ValueError("pstore must be a contiguous uint8 tensor")
        if host_offsets is not None:
            ho = torch.as_tensor(host_offsets, dtype=torch.int64, device="cpu").contiguous()
            if ho.numel() != B + 1:
                raise ValueError("host_offsets must hold B + 1 offsets")
            _check(library().hstu_attn_bwd_pstore_chunked(
                _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                _ptr(seq_offsets), ctypes.c_void_p(ho.data_ptr()), B, total, H, D, _ptr(func),
                nfunc, float(alpha), int(max_len), _ptr(ws), ws.numel(), _ptr(pstore),
                pstore.numel(), _stream(k.device)))
            return dq, dk, dv
        _check(library().hstu_attn_bwd_pstore(
            _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(seq_offsets), B, total, H, D, _ptr(func), nfunc, float(alpha), int(max_len),
            _ptr(ws), ws.numel(), _ptr(pstore), pstore.numel(), _stream(k.device)))
        return dq, dk, dv
    _check(library().hstu_attn_bwd(
        code, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(seq_offsets), B, total, H, D, _ptr(func), nfunc, float(alpha), int(max_len),
        _ptr(target_rows), _ptr(ws), ws.numel(), _stream(k.device)))
    return dq, dk, dv


def attn_bwd_atomic(q, k, v, dout, seq_offsets, func, alpha, max_len, dq_accum=None):
    """Backward with dQ accumulated by fp32 atomics in the key-owner pass
    (bf16, D = 128, full-length mode): dk and dv as attn_bwd (bitwise), dq up
    to the order of its fp32 additions (not bitwise repeatable).  ``dq_accum``
    is an optional float32 CUDA tensor of at least total*H*D elements used as
    the accumulator (allocated here when not given)."""
    B, total, H, D, nfunc = _common(q, k, seq_offsets, func, None)
    for t in (q, k, v, dout):
        if not t.is_contiguous() or t.dtype != k.dtype:
            raise ValueError("q, k, v, dout must be contiguous and share a dtype")
    if _dtype_code(k) != HSTU_BF16:
        raise ValueError("the atomic-dQ backward needs bf16")
    if dq_accum is None:
        dq_accum = torch.empty((total, H, D), dtype=torch.float32, device=k.device)
    if dq_accum.dtype != torch.float32 or not dq_accum.is_contiguous():
        raise ValueError("dq_accum must be a contiguous float32 tensor")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws_bytes = workspace_size(1, B, total, H, D, nfunc, False)
    ws = _workspace(ws_bytes, k.device)
    _check(library().hstu_attn_bwd_atomic(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(seq_offsets), B, total, H, D, _ptr(func), nfunc, float(alpha), int(max_len),
        _ptr(ws), ws.numel(), _ptr(dq_accum), dq_accum.numel() * 4, _stream(k.device)))
    return dq, dk, dv


def visible_counts(seq_offsets, func, total=None, target_rows=None):
    """Per-row visible-column counts (int32) and their sum (int64 tensor)."""
    B = seq_offsets.numel() - 1
    total = func.shape[1] if total is None else int(total)
    n = B if target_rows is not None else total
    counts = torch.empty(n, dtype=torch.int32, device=func.device)
    tot = torch.empty(1, dtype=torch.int64, device=func.device)
    _check(library().hstu_attn_visible_counts(
        _ptr(seq_offsets), B, total, _ptr(func), func.shape[0], _ptr(target_rows), _ptr(counts),
        _ptr(tot), _stream(func.device)))
    return counts, tot


def check_inputs(seq_offsets, total, target_rows=None):
    """Validate device-resident offsets / target rows (synchronizes)."""
    B = seq_offsets.numel() - 1
    ws = _workspace(workspace_size(0, B, total, 1, 128, 1, 0), seq_offsets.device)
    _check(library().hstu_attn_check_inputs(_ptr(seq_offsets), B, int(total), _ptr(target_rows),
                                            _ptr(ws), ws.numel(), _stream(seq_offsets.device)))


def profile_enable(on: bool = True) -> bool:
    """Turn per-kernel HIP-event timing on or off; returns the previous state."""
    return bool(library().hstu_profile_enable(1 if on else 0))


def profile_reset() -> None:
    library().hstu_profile_reset()


def profile_read() -> dict:
    """{kernel_name: (launches, total_ms)} accumulated since the last reset."""
    lib = library()
    need = lib.hstu_profile_read(None, 0)
    buf = ctypes.create_string_buffer(int(need) + 64)
    lib.hstu_profile_read(buf, len(buf))
    out = {}
    for line in buf.value.decode().splitlines():
        name, count, ms = line.split()
        out[name] = (int(count), float(ms))
    return out


class HstuAttention(torch.autograd.Function):
    """Autograd wrapper: forward = attn_fwd, backward = attn_bwd (nothing saved
    but the inputs: HSTU attention has no softmax statistics to keep).  With
    ``pstore`` (and optionally ``host_offsets``) the backward is the stored-P
    one, as in attn_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, seq_offsets, func, alpha, max_len, target_rows, pstore,
                host_offsets):
        ctx.save_for_backward(q, k, v, seq_offsets, func, target_rows)
        ctx.alpha, ctx.max_len = alpha, max_len
        ctx.pstore, ctx.host_offsets = pstore, host_offsets
        return attn_fwd(q, k, v, seq_offsets, func, alpha, max_len, target_rows)

    @staticmethod
    def backward(ctx, dout):
        q, k, v, seq_offsets, func, target_rows = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, dout.contiguous(), seq_offsets, func, ctx.alpha,
                              ctx.max_len, target_rows, pstore=ctx.pstore,
                              host_offsets=ctx.host_offsets)
        return dq, dk, dv, None, None, None, None, None, None, None


def hstu_attention(q, k, v, seq_offsets, func, alpha, max_len, target_rows=None, pstore=None,
                   host_offsets=None):
    """HSTU attention with autograd.  ``pstore``: a uint8 CUDA buffer for the
    stored-P backward (bf16, D = 128, full-length), of pstore_bytes() bytes,
    or smaller when ``host_offsets`` (a CPU copy of seq_offsets) is given."""
    return HstuAttention.apply(q, k, v, seq_offsets, func, alpha, max_len, target_rows, pstore,
                               host_offsets)
