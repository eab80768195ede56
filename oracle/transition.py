"""fp64 CPU oracle for the fused SwiGLU transition (test infrastructure).

ORACLE -- TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import this module.  It imports nothing
from the HIP library or its binding and shares no code with them.

What it computes (MegaFold, gist.science technical summary, Methodik section 3
"EvoFusion": layer normalisation, linear projections and SwiGLU activations are
fused so that intermediates are not materialised in HBM; the pages give no
formulas).  The plainest reading is the gated transition of a pair or MSA
tensor: layer norm, two bias-free expansions to n*C hidden units, the SwiGLU
gate silu(a) * b, and a bias-free projection back to C channels:

  y   = layer_norm(x; gamma, beta, eps)                 (over the C channels)
  a   = y @ w_a^T,  b = y @ w_b^T                       ([T, n*C] each)
  h   = silu(a) * b,  silu(a) = a * sigmoid(a)
  out = h @ w_out^T                                     ([T, C])

Backward, for the loss L = sum out * dout:

  dh     = dout @ w_out,            dw_out = dout^T @ h
  da     = dh * b * silu'(a),       silu'(a) = sigmoid(a) * (1 + a * (1 - sigmoid(a)))
  db     = dh * silu(a)
  dy     = da @ w_a + db @ w_b,     dw_a = da^T @ y,  dw_b = db^T @ y
  dgamma = sum_t dy * xhat,  dbeta = sum_t dy,
  dx     = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat)),  g = dy * gamma

Parity pins (CPU tests): a hand-derived two-channel example, closed forms of
silu and its derivative, the gate direction (silu applied to a, not b),
linearity in w_b and w_out, and central finite differences of every gradient.
"""
from __future__ import annotations

import numpy as np

from .ln_proj import _f64, layer_norm


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    return a * sigmoid(a)


def silu_grad(a):
    s = sigmoid(a)
    return s * (1.0 + a * (1.0 - s))


def transition_fwd(x, gamma, beta, eps, w_a, w_b, w_out):
    """Returns dict out [A, B, C], mean, rstd [A, B]."""
    x = _f64(x)
    y, _xhat, mean, rstd = layer_norm(x, gamma, beta, eps)
    a = y @ _f64(w_a).T
    b = y @ _f64(w_b).T
    h = silu(a) * b
    return {"out": h @ _f64(w_out).T, "mean": mean, "rstd": rstd}


def transition_bwd(x, gamma, beta, eps, w_a, w_b, w_out, dout):
    """Gradients of L = sum out * dout: dict dx, dgamma, dbeta, dw_a, dw_b, dw_out."""
    x = _f64(x)
    A, B, C = x.shape
    T = A * B
    wa, wb, wo = _f64(w_a), _f64(w_b), _f64(w_out)
    y, xhat, _mean, rstd = layer_norm(x, gamma, beta, eps)
    y2, xh2 = y.reshape(T, C), xhat.reshape(T, C)
    a = y2 @ wa.T
    b = y2 @ wb.T
    h = silu(a) * b
    do = _f64(dout).reshape(T, C)
    dh = do @ wo
    da = dh * b * silu_grad(a)
    db = dh * silu(a)
    dy = da @ wa + db @ wb
    g = dy * _f64(gamma)
    dx = rstd.reshape(T, 1) * (g - g.mean(axis=1, keepdims=True)
                               - xh2 * (g * xh2).mean(axis=1, keepdims=True))
    return {"dx": dx.reshape(A, B, C), "dgamma": (dy * xh2).sum(axis=0), "dbeta": dy.sum(axis=0),
            "dw_a": da.T @ y2, "dw_b": db.T @ y2, "dw_out": do.T @ h}
