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
