"""Python face of the EvoAttention C ABI: argument marshalling only.

Every step of the computation runs in the HIP library (libevoattn.so); this
module checks tensor properties, allocates outputs and workspace with torch's
caching allocator, and passes raw device pointers plus torch's current stream.

Layouts (kernel frame, see include/evoattn.h): q, k, v, dout are [R, N, H, d]
when transpose is False and [N, R, H, d] when True; bias is [H, N, N]; mask is
[R, N] fp32 additive; lse is [R, H, N] fp32.
"""
from __future__ import annotations

import torch

from . import _lib

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


def _dims(q: torch.Tensor, transpose: bool):
    if q.dim() != 4:
        raise ValueError(f"q must be 4-D [R,N,H,d] (or [N,R,H,d] transposed), got {tuple(q.shape)}")
    a, b, H, D = q.shape
    R, N = (b, a) if transpose else (a, b)
    return R, N, H, D


def _check(t, name, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def evoattn_fwd_workspace_bytes(rows, n, heads, head_dim, dtype=torch.bfloat16) -> int:
    return int(_lib.load().evoattn_fwd_workspace_bytes(rows, n, heads, head_dim, _DTYPES[dtype]))


def evoattn_bwd_workspace_bytes(rows, n, heads, head_dim, dtype=torch.bfloat16) -> int:
    return int(_lib.load().evoattn_bwd_workspace_bytes(rows, n, heads, head_dim, _DTYPES[dtype]))


def evoattn_fwd(q, k, v, bias=None, mask=None, transpose=False, need_lse=True, out=None, lse_out=None):
    """Forward.  Returns (o, lse); lse is None when need_lse is False."""
    lib = _lib.load()
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    R, N, H, D = _dims(q, transpose)
    dev = q.device
    _check(q, "q", q.shape, q.dtype, dev)
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(bias, "bias", (H, N, N), q.dtype, dev, optional=True)
    _check(mask, "mask", (R, N), torch.float32, dev, optional=True)
    o = out if out is not None else torch.empty_like(q)
    _check(o, "out", q.shape, q.dtype, dev)
    lse = None
    if need_lse:
        lse = lse_out if lse_out is not None else torch.empty((R, H, N), dtype=torch.float32, device=dev)
        _check(lse, "lse_out", (R, H, N), torch.float32, dev)
    ws_bytes = int(lib.evoattn_fwd_workspace_bytes(R, N, H, D, _DTYPES[q.dtype]))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = lib.evoattn_fwd(R, N, H, D, _DTYPES[q.dtype], int(bool(transpose)),
                         _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(o), _ptr(lse),
                         _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(st, "evoattn_fwd")
    return o, lse


def evoattn_fwd_noalloc(q, k, v, bias=None, mask=None, transpose=False, out=None, lse_out=None):
    """Forward through the entry point that allocates nothing (its scratch is a static
    device array of the library).  Pass `out` and `lse_out` to allocate nothing here
    either; otherwise they are created.  Returns (o, lse)."""
    lib = _lib.load()
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    R, N, H, D = _dims(q, transpose)
    dev = q.device
    _check(q, "q", q.shape, q.dtype, dev)
    _check(k, "k", q.shape, q.dtype, dev)
    _check(v, "v", q.shape, q.dtype, dev)
    _check(bias, "bias", (H, N, N), q.dtype, dev, optional=True)
    _check(mask, "mask", (R, N), torch.float32, dev, optional=True)
    o = out if out is not None else torch.empty_like(q)
    _check(o, "out", q.shape, q.dtype, dev)
    lse = lse_out if lse_out is not None else torch.empty((R, H, N), dtype=torch.float32, device=dev)
    _check(lse, "lse_out", (R, H, N), torch.float32, dev)
    st = lib.evoattn_fwd_noalloc(R, N, H, D, _DTYPES[q.dtype], int(bool(transpose)),
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(o), _ptr(lse), _stream(dev))
    _lib.check(st, "evoattn_fwd_noalloc")
    return o, lse


def evoattn_bwd(q, k, v, bias, mask, o, lse, dout, transpose=False, need_dbias=True, workspace=None):
    """Backward of sum(o * dout).  Returns (dq, dk, dv, dbias); dbias is fp32 [H,N,N] or None."""
    lib = _lib.load()
    R, N, H, D = _dims(q, transpose)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check(t, name, q.shape, q.dtype, dev)
    _check(bias, "bias", (H, N, N), q.dtype, dev, optional=True)
    _check(mask, "mask", (R, N), torch.float32, dev, optional=True)
    _check(lse, "lse", (R, H, N), torch.float32, dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dbias = torch.empty((H, N, N), dtype=torch.float32, device=dev) if need_dbias else None
    ws_bytes = int(lib.evoattn_bwd_workspace_bytes(R, N, H, D, _DTYPES[q.dtype]))
    ws = workspace
    if ws is None or ws.numel() < ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = lib.evoattn_bwd(R, N, H, D, _DTYPES[q.dtype], int(bool(transpose)),
                         _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask), _ptr(o), _ptr(lse), _ptr(dout),
                         _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(st, "evoattn_bwd")
    return dq, dk, dv, dbias


class EvoAttnFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, bias, mask, transpose):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        bias = None if bias is None else bias.contiguous()
        o, lse = evoattn_fwd(q, k, v, bias, mask, transpose)
        ctx.save_for_backward(q, k, v, bias, mask, o, lse)
        ctx.transpose = transpose
        ctx.has_bias = bias is not None
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, bias, mask, o, lse = ctx.saved_tensors
        dq, dk, dv, dbias = evoattn_bwd(q, k, v, bias, mask, o, lse, dout.contiguous(), ctx.transpose,
                                        need_dbias=ctx.has_bias and ctx.needs_input_grad[3])
        if dbias is not None:
            dbias = dbias.to(bias.dtype)
        return dq, dk, dv, dbias, None, None


def evoattn(q, k, v, bias=None, mask=None, transpose=False):
    """Differentiable pair-biased 3D attention; returns o in q's layout and dtype."""
    return EvoAttnFunction.apply(q, k, v, bias, mask, bool(transpose))
