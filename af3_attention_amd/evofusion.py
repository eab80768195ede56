"""Python face of the fused layer norm + projections C ABI (include/evofusion.h):
argument marshalling only.  The computation runs in libevoattn.so.

x is [A, B, C] (pair tensor: A = B = N; MSA tensor: A = S, B = N); w_qkv is
[3*H*d, C] (a torch Linear weight: rows q, then k, then v, each h*d + e);
w_bias is [H, C]; gamma and beta are fp32 [C].  Outputs q, k, v are
[A, B, H, d] in x's token order and bias is [H, A, B] (bias[h, a, b] from token
(b, a) when bias_transpose is set, the ending node's frame).
"""
from __future__ import annotations

import torch

from . import _lib
from .evoattn import _DTYPES, _check, _ptr, _stream


def ln_proj_fwd(x, gamma, beta, w_qkv=None, w_bias=None, *, heads: int, head_dim: int,
                bias_transpose: bool = False, eps: float = 1e-5, need_stats: bool = True):
    """Returns dict q, k, v (or None), bias (or None), mean, rstd (fp32 [A*B], or None)."""
    lib = _lib.load()
    if x.dim() != 3:
        raise ValueError(f"x must be 3-D [A, B, C], got {tuple(x.shape)}")
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    A, B, C = x.shape
    dev = x.device
    hd = heads * head_dim
    _check(x, "x", x.shape, x.dtype, dev)
    _check(gamma, "gamma", (C,), torch.float32, dev)
    _check(beta, "beta", (C,), torch.float32, dev)
    _check(w_qkv, "w_qkv", (3 * hd, C), x.dtype, dev, optional=True)
    _check(w_bias, "w_bias", (heads, C), x.dtype, dev, optional=True)
    out = {"q": None, "k": None, "v": None, "bias": None, "mean": None, "rstd": None}
    if w_qkv is not None:
        for n in ("q", "k", "v"):
            out[n] = torch.empty((A, B, heads, head_dim), dtype=x.dtype, device=dev)
    if w_bias is not None:
        out["bias"] = torch.empty((heads, A, B), dtype=x.dtype, device=dev)
    if need_stats:
        out["mean"] = torch.empty(A * B, dtype=torch.float32, device=dev)
        out["rstd"] = torch.empty(A * B, dtype=torch.float32, device=dev)
    st = lib.evoattn_ln_proj_fwd(A, B, C, heads, head_dim, _DTYPES[x.dtype], int(bool(bias_transpose)),
                                 float(eps), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(w_qkv), _ptr(w_bias),
                                 _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["bias"]),
                                 _ptr(out["mean"]), _ptr(out["rstd"]), _stream(dev))
    _lib.check(st, "evoattn_ln_proj_fwd")
    return out


def ln_proj_bwd_workspace_bytes(a, b, channels, heads, head_dim, dtype=torch.bfloat16, with_qkv=True,
                                with_bias=True) -> int:
    return int(_lib.load().evoattn_ln_proj_bwd_workspace_bytes(a, b, channels, heads, head_dim, _DTYPES[dtype],
                                                                int(bool(with_qkv)), int(bool(with_bias))))


def ln_proj_bwd(x, gamma, beta, w_qkv, w_bias, mean, rstd, dq=None, dk=None, dv=None, dbias=None, *,
                heads: int, head_dim: int, bias_transpose: bool = False, workspace=None):
    """Gradients of sum(q*dq) + sum(k*dk) + sum(v*dv) + sum(bias*dbias) through ln_proj_fwd.

    dbias is fp32 [H, A, B] (as evoattn_bwd returns it).  Returns dict dx (x's dtype),
    dgamma, dbeta (fp32 [C]), dw_qkv (fp32 [3Hd, C] or None), dw_bias (fp32 [H, C] or None)."""
    lib = _lib.load()
    A, B, C = x.shape
    dev = x.device
    hd = heads * head_dim
    _check(x, "x", x.shape, x.dtype, dev)
    _check(gamma, "gamma", (C,), torch.float32, dev)
    _check(beta, "beta", (C,), torch.float32, dev)
    _check(w_qkv, "w_qkv", (3 * hd, C), x.dtype, dev, optional=True)
    _check(w_bias, "w_bias", (heads, C), x.dtype, dev, optional=True)
    _check(mean, "mean", (A * B,), torch.float32, dev)
    _check(rstd, "rstd", (A * B,), torch.float32, dev)
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, n, (A, B, heads, head_dim), x.dtype, dev, optional=w_qkv is None)
    _check(dbias, "dbias", (heads, A, B), torch.float32, dev, optional=w_bias is None)
    out = {"dx": torch.empty_like(x),
           "dgamma": torch.empty(C, dtype=torch.float32, device=dev),
           "dbeta": torch.empty(C, dtype=torch.float32, device=dev),
           "dw_qkv": None if w_qkv is None else torch.empty((3 * hd, C), dtype=torch.float32, device=dev),
           "dw_bias": None if w_bias is None else torch.empty((heads, C), dtype=torch.float32, device=dev)}
    ws_bytes = ln_proj_bwd_workspace_bytes(A, B, C, heads, head_dim, x.dtype, w_qkv is not None, w_bias is not None)
    ws = workspace
    if ws is None or ws.numel() < ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.evoattn_ln_proj_bwd(A, B, C, heads, head_dim, _DTYPES[x.dtype], int(bool(bias_transpose)),
                                 _ptr(x), _ptr(gamma), _ptr(beta), _ptr(w_qkv), _ptr(w_bias), _ptr(mean),
                                 _ptr(rstd), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(out["dx"]),
                                 _ptr(out["dgamma"]), _ptr(out["dbeta"]), _ptr(out["dw_qkv"]),
                                 _ptr(out["dw_bias"]), _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(st, "evoattn_ln_proj_bwd")
    return out


class LNProjFunction(torch.autograd.Function):
    """Differentiable fused layer norm + projections; outputs (q, k, v, bias), None where absent."""

    @staticmethod
    def forward(ctx, x, gamma, beta, w_qkv, w_bias, heads, head_dim, bias_transpose, eps):
        x = x.contiguous()
        out = ln_proj_fwd(x, gamma, beta, w_qkv, w_bias, heads=heads, head_dim=head_dim,
                          bias_transpose=bias_transpose, eps=eps)
        ctx.save_for_backward(x, gamma, beta, w_qkv, w_bias, out["mean"], out["rstd"])
        ctx.cfg = (heads, head_dim, bias_transpose)
        return out["q"], out["k"], out["v"], out["bias"]

    @staticmethod
    def backward(ctx, dq, dk, dv, dbias):
        x, gamma, beta, w_qkv, w_bias, mean, rstd = ctx.saved_tensors
        heads, head_dim, bt = ctx.cfg
        shape = (x.shape[0], x.shape[1], heads, head_dim)
        if w_qkv is not None:
            dq, dk, dv = (torch.zeros(shape, dtype=x.dtype, device=x.device) if g is None else g.contiguous()
                          for g in (dq, dk, dv))
        if w_bias is not None:
            dbias = (torch.zeros((heads, x.shape[0], x.shape[1]), dtype=torch.float32, device=x.device)
                     if dbias is None else dbias.float().contiguous())
        g = ln_proj_bwd(x, gamma, beta, w_qkv, w_bias, mean, rstd, dq, dk, dv, dbias, heads=heads,
                        head_dim=head_dim, bias_transpose=bt)
        dwq = None if g["dw_qkv"] is None else g["dw_qkv"].to(w_qkv.dtype)
        dwb = None if g["dw_bias"] is None else g["dw_bias"].to(w_bias.dtype)
        return g["dx"], g["dgamma"], g["dbeta"], dwq, dwb, None, None, None, None


def ln_proj(x, gamma, beta, w_qkv=None, w_bias=None, *, heads: int, head_dim: int, bias_transpose: bool = False,
            eps: float = 1e-5):
    """Differentiable layer norm + projections: returns (q, k, v, bias), None where absent."""
    return LNProjFunction.apply(x, gamma, beta, w_qkv, w_bias, heads, head_dim, bool(bias_transpose), float(eps))


# ---------------------------------------------------------------- transition

def transition_fwd(x, gamma, beta, w_a, w_b, w_out, *, eps: float = 1e-5, need_stats: bool = True):
    """SwiGLU transition: returns dict out ([A, B, C], x's dtype), mean, rstd (fp32 [A*B] or None)."""
    lib = _lib.load()
    if x.dim() != 3:
        raise ValueError(f"x must be 3-D [A, B, C], got {tuple(x.shape)}")
    A, B, C = x.shape
    dev = x.device
    hidden = w_a.shape[0] if w_a.dim() == 2 else -1
    if hidden % C != 0 or hidden <= 0:
        raise ValueError(f"w_a must be [n*C, C], got {tuple(w_a.shape)}")
    _check(x, "x", x.shape, x.dtype, dev)
    _check(gamma, "gamma", (C,), torch.float32, dev)
    _check(beta, "beta", (C,), torch.float32, dev)
    _check(w_a, "w_a", (hidden, C), x.dtype, dev)
    _check(w_b, "w_b", (hidden, C), x.dtype, dev)
    _check(w_out, "w_out", (C, hidden), x.dtype, dev)
    out = {"out": torch.empty_like(x), "mean": None, "rstd": None}
    if need_stats:
        out["mean"] = torch.empty(A * B, dtype=torch.float32, device=dev)
        out["rstd"] = torch.empty(A * B, dtype=torch.float32, device=dev)
    st = lib.evoattn_transition_fwd(A, B, C, hidden // C, _DTYPES[x.dtype], float(eps), _ptr(x), _ptr(gamma),
                                    _ptr(beta), _ptr(w_a), _ptr(w_b), _ptr(w_out), _ptr(out["out"]),
                                    _ptr(out["mean"]), _ptr(out["rstd"]), _stream(dev))
    _lib.check(st, "evoattn_transition_fwd")
    return out


def transition_bwd_workspace_bytes(a, b, channels, expansion, dtype=torch.bfloat16) -> int:
    return int(_lib.load().evoattn_transition_bwd_workspace_bytes(a, b, channels, expansion, _DTYPES[dtype]))


def transition_bwd(x, gamma, beta, w_a, w_b, w_out, mean, rstd, dout, *, workspace=None):
    """Gradients of sum(out * dout): dict dx (x's dtype), dgamma, dbeta (fp32 [C]),
    dw_a, dw_b (fp32 [n*C, C]), dw_out (fp32 [C, n*C])."""
    lib = _lib.load()
    A, B, C = x.shape
    dev = x.device
    hidden = w_a.shape[0]
    _check(x, "x", x.shape, x.dtype, dev)
    _check(gamma, "gamma", (C,), torch.float32, dev)
    _check(beta, "beta", (C,), torch.float32, dev)
    _check(w_a, "w_a", (hidden, C), x.dtype, dev)
    _check(w_b, "w_b", (hidden, C), x.dtype, dev)
    _check(w_out, "w_out", (C, hidden), x.dtype, dev)
    _check(mean, "mean", (A * B,), torch.float32, dev)
    _check(rstd, "rstd", (A * B,), torch.float32, dev)
    _check(dout, "dout", x.shape, x.dtype, dev)
    out = {"dx": torch.empty_like(x), "dgamma": torch.empty(C, dtype=torch.float32, device=dev),
           "dbeta": torch.empty(C, dtype=torch.float32, device=dev),
           "dw_a": torch.empty((hidden, C), dtype=torch.float32, device=dev),
           "dw_b": torch.empty((hidden, C), dtype=torch.float32, device=dev),
           "dw_out": torch.empty((C, hidden), dtype=torch.float32, device=dev)}
    n = hidden // C
    ws_bytes = transition_bwd_workspace_bytes(A, B, C, n, x.dtype)
    ws = workspace
    if ws is None or ws.numel() < ws_bytes:
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = lib.evoattn_transition_bwd(A, B, C, n, _DTYPES[x.dtype], _ptr(x), _ptr(gamma), _ptr(beta), _ptr(w_a),
                                    _ptr(w_b), _ptr(w_out), _ptr(mean), _ptr(rstd), _ptr(dout), _ptr(out["dx"]),
                                    _ptr(out["dgamma"]), _ptr(out["dbeta"]), _ptr(out["dw_a"]), _ptr(out["dw_b"]),
                                    _ptr(out["dw_out"]), _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(st, "evoattn_transition_bwd")
    return out


class TransitionFunction(torch.autograd.Function):
    """Differentiable fused SwiGLU transition."""

    @staticmethod
    def forward(ctx, x, gamma, beta, w_a, w_b, w_out, eps):
        x = x.contiguous()
        r = transition_fwd(x, gamma, beta, w_a, w_b, w_out, eps=eps)
        ctx.save_for_backward(x, gamma, beta, w_a, w_b, w_out, r["mean"], r["rstd"])
        return r["out"]

    @staticmethod
    def backward(ctx, dout):
        x, gamma, beta, w_a, w_b, w_out, mean, rstd = ctx.saved_tensors
        g = transition_bwd(x, gamma, beta, w_a, w_b, w_out, mean, rstd, dout.contiguous())
        return (g["dx"], g["dgamma"], g["dbeta"], g["dw_a"].to(w_a.dtype), g["dw_b"].to(w_b.dtype),
                g["dw_out"].to(w_out.dtype), None)


def transition(x, gamma, beta, w_a, w_b, w_out, *, eps: float = 1e-5):
    """Differentiable fused SwiGLU transition: out = (silu(y w_a^T) * y w_b^T) w_out^T, y = LN(x)."""
    return TransitionFunction.apply(x, gamma, beta, w_a, w_b, w_out, float(eps))
