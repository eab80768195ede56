"""fp64 CPU oracle for the fused LayerNorm + linear projections that feed the
attention (test infrastructure).

ORACLE -- TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import this module.  It imports nothing
from the HIP library or its binding and shares no code with them.

What it computes (MegaFold, gist.science technical summary, Methodik section 3
"EvoFusion"): the pages name layer normalisation followed by linear projections
as one of the fused operator groups; the fused kernel must not write the
normalised N x N tensor to HBM between the two.  The pages give no formulas,
so this file writes out the plainest reading, the textbook layer norm over the
channels of each token of the pair (or MSA) tensor followed by bias-free
projections into the attention's inputs:

  x        : [A, B, c], token t = (a, b); c channels
  mean[t]  = (1/c) sum_c x[t, c]
  var[t]   = (1/c) sum_c (x[t, c] - mean[t])^2          (biased variance)
  rstd[t]  = 1 / sqrt(var[t] + eps)
  xhat     = (x - mean) * rstd
  y        = xhat * gamma + beta                        (per-channel affine)
  qkv[t,o] = sum_c y[t, c] w_qkv[o, c],  o < 3*H*d      (rows: q, then k, then v;
                                                         inside each, o = h*d + e)
  q[a, b, h, e] = qkv[t, h*d + e], k = ... + H*d, v = ... + 2*H*d
  pb[t, h] = sum_c y[t, c] w_bias[h, c]                 (pair bias, needs A == B)
  bias[h, a, b] = pb[(a, b), h]     when bias_transpose == 0
  bias[h, a, b] = pb[(b, a), h]     when bias_transpose == 1 (ending node: the
                                     kernel frame's query is the pair tensor's
                                     column index)

Backward, for the loss  L = sum q*dq + sum k*dk + sum v*dv + sum bias*dbias:

  G[t, o]   = upstream gradient of qkv and pb (dq|dk|dv|dbias gathered per token)
  dy        = G @ [w_qkv; w_bias]                       (gradient of y)
  dw        = G^T @ y                                   (gradients of the weights)
  dgamma    = sum_t dy * xhat,   dbeta = sum_t dy
  g         = dy * gamma
  dx        = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat))

Parity pins (CPU tests): closed forms for c = 2 and for tokens that are an
affine image of one standardised vector, the eps placement, mean 0 / variance 1
of xhat, invariance to per-token shift and positive scale, the output layout
(selection-matrix weights), and central finite differences of every gradient.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def layer_norm(x, gamma, beta, eps):
    """Textbook layer norm over the last axis.  Returns (y, xhat, mean, rstd)."""
    x = _f64(x)
    mean = x.mean(axis=-1)
    cen = x - mean[..., None]
    var = (cen * cen).mean(axis=-1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = cen * rstd[..., None]
    y = xhat * _f64(gamma) + _f64(beta)
    return y, xhat, mean, rstd


def _bias_to_tokens(bias, bias_transpose):
    """[H, A, B] kernel-frame bias -> [A, B, H] token order (inverse of the output map)."""
    b = bias.transpose(0, 2, 1) if bias_transpose else bias
    return np.moveaxis(b, 0, -1)


def ln_proj_fwd(x, gamma, beta, eps, w_qkv, w_bias, heads, head_dim, bias_transpose=0):
    """Returns dict q, k, v ([A, B, H, d] or None), bias ([H, A, B] or None), mean, rstd ([A, B])."""
    x = _f64(x)
    A, B, c = x.shape
    y, _xhat, mean, rstd = layer_norm(x, gamma, beta, eps)
    out = {"q": None, "k": None, "v": None, "bias": None, "mean": mean, "rstd": rstd}
    hd = heads * head_dim
    if w_qkv is not None:
        w = _f64(w_qkv)
        assert w.shape == (3 * hd, c)
        qkv = y @ w.T  # [A, B, 3*H*d]
        for i, name in enumerate(("q", "k", "v")):
            out[name] = qkv[..., i * hd:(i + 1) * hd].reshape(A, B, heads, head_dim).copy()
    if w_bias is not None:
        assert A == B, "the pair bias needs a square pair tensor"
        wb = _f64(w_bias)
        assert wb.shape == (heads, c)
        pb = y @ wb.T  # [A, B, H]
        bias = np.moveaxis(pb, -1, 0)  # [H, A, B]
        if bias_transpose:
            bias = bias.transpose(0, 2, 1)
        out["bias"] = np.ascontiguousarray(bias)
    return out


def ln_proj_bwd(x, gamma, beta, eps, w_qkv, w_bias, heads, head_dim, bias_transpose,
                dq=None, dk=None, dv=None, dbias=None):
    """Gradients of L = sum q*dq + sum k*dk + sum v*dv + sum bias*dbias.

    Returns dict dx [A, B, c], dgamma [c], dbeta [c], dw_qkv [3Hd, c] (or None),
    dw_bias [H, c] (or None)."""
    x = _f64(x)
    A, B, c = x.shape
    T = A * B
    y, xhat, _mean, rstd = layer_norm(x, gamma, beta, eps)
    y2 = y.reshape(T, c)
    dy = np.zeros((T, c))
    res = {"dw_qkv": None, "dw_bias": None}
    if w_qkv is not None:
        G = np.concatenate([_f64(g).reshape(T, heads * head_dim) for g in (dq, dk, dv)], axis=1)
        dy += G @ _f64(w_qkv)
        res["dw_qkv"] = G.T @ y2
    if w_bias is not None:
        Gb = _bias_to_tokens(_f64(dbias), bias_transpose).reshape(T, heads)
        dy += Gb @ _f64(w_bias)
        res["dw_bias"] = Gb.T @ y2
    xh2 = xhat.reshape(T, c)
    res["dgamma"] = (dy * xh2).sum(axis=0)
    res["dbeta"] = dy.sum(axis=0)
    g = dy * _f64(gamma)
    dx = rstd.reshape(T, 1) * (g - g.mean(axis=1, keepdims=True)
                               - xh2 * (g * xh2).mean(axis=1, keepdims=True))
    res["dx"] = dx.reshape(A, B, c)
    return res
