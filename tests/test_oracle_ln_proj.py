"""Pins for the fp64 oracle of layer norm + projections (EvoFusion's first group),
independent of the oracle's own code.

The pages (MegaFold, gist.science technical summary, Methodik section 3
"EvoFusion") name the operators but print no formulas; the oracle follows the
textbook layer norm (biased variance, eps added to the variance, per-channel
gain and offset) and bias-free projections.  These tests fix it by hand-derived
values, invariants of normalisation, the output layout seen through
selection-matrix weights, and central finite differences of its forward.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import generate_proj


def fwd(x, gamma, beta, eps, w_qkv, w_bias, H, D, bt=0):
    return oracle.ln_proj_fwd(np.asarray(x, float), np.asarray(gamma, float), np.asarray(beta, float), eps,
                              None if w_qkv is None else np.asarray(w_qkv, float),
                              None if w_bias is None else np.asarray(w_bias, float), H, D, bt)


# ---------------------------------------------------------------- hand-derived values

def test_two_channel_token_by_hand():
    """x = [3, 1]: mean 2, deviations [1, -1], variance 1, so xhat = [1, -1] (eps = 0).
    gamma = [2, 3], beta = [0.5, -1] give y = [2.5, -4].  With H = 1, d = 2 and the
    weight rows below, q = [2.5, -4], k = [-1.5, 6.5], v = [5, 2], bias = 0.25."""
    w_qkv = [[1, 0], [0, 1], [1, 1], [1, -1], [2, 0], [0, -0.5]]
    out = fwd([[[3.0, 1.0]]], [2, 3], [0.5, -1], 0.0, w_qkv, [[0.5, 0.25]], 1, 2)
    np.testing.assert_allclose(out["q"].ravel(), [2.5, -4], atol=1e-14)
    np.testing.assert_allclose(out["k"].ravel(), [-1.5, 6.5], atol=1e-14)
    np.testing.assert_allclose(out["v"].ravel(), [5, 2], atol=1e-14)
    np.testing.assert_allclose(out["bias"].ravel(), [0.25], atol=1e-14)
    np.testing.assert_allclose(out["mean"].ravel(), [2.0], atol=1e-14)
    np.testing.assert_allclose(out["rstd"].ravel(), [1.0], atol=1e-14)


def test_eps_and_biased_variance_by_hand():
    """x = [0, 0, 0, 4]: mean 1, deviations [-1, -1, -1, 3], biased variance 12/4 = 3;
    with eps = 1, rstd = 1/sqrt(4) = 1/2 and xhat = [-0.5, -0.5, -0.5, 1.5].
    (An unbiased variance would give 1/sqrt(5); eps on the standard deviation
    1/(sqrt(3) + 1).)  x = [-1, 1] with eps = 0.25: xhat = [-1, 1] / sqrt(1.25)."""
    y, xhat, mean, rstd = oracle.layer_norm(np.array([[0.0, 0, 0, 4]]), np.ones(4), np.zeros(4), 1.0)
    np.testing.assert_allclose(xhat.ravel(), [-0.5, -0.5, -0.5, 1.5], atol=1e-15)
    np.testing.assert_allclose(rstd, [0.5], atol=1e-15)
    np.testing.assert_allclose(mean, [1.0], atol=1e-15)
    _, xhat2, _, _ = oracle.layer_norm(np.array([[-1.0, 1.0]]), np.ones(2), np.zeros(2), 0.25)
    np.testing.assert_allclose(xhat2.ravel(), [-1 / 1.25 ** 0.5, 1 / 1.25 ** 0.5], atol=1e-15)


def test_pair_bias_orientation_by_hand():
    """Two-channel tokens normalise to [1, -1] when x0 > x1 and to [-1, 1] otherwise
    (eps = 0).  With gamma = 1, beta = 0 and w_bias = [[1, 0]] the bias of token
    (a, b) is +1 or -1.  Tokens (0,0)=[1,0], (0,1)=[0,1], (1,0)=[5,2], (1,1)=[2,5]
    give pb = [[1, -1], [1, -1]] by token; transposed it reads [[1, 1], [-1, -1]]."""
    x = [[[1.0, 0.0], [0.0, 1.0]], [[5.0, 2.0], [2.0, 5.0]]]
    o0 = fwd(x, [1, 1], [0, 0], 0.0, None, [[1.0, 0.0]], 1, 2, 0)
    o1 = fwd(x, [1, 1], [0, 0], 0.0, None, [[1.0, 0.0]], 1, 2, 1)
    np.testing.assert_allclose(o0["bias"][0], [[1, -1], [1, -1]], atol=1e-14)
    np.testing.assert_allclose(o1["bias"][0], [[1, 1], [-1, -1]], atol=1e-14)
    assert o0["q"] is None and o0["k"] is None and o0["v"] is None


# ---------------------------------------------------------------- invariants

def standardised(rng, shape):
    """Random vectors rescaled to mean 0 and biased variance 1 along the last axis."""
    u = rng.standard_normal(shape)
    u -= u.mean(axis=-1, keepdims=True)
    u /= np.sqrt((u * u).mean(axis=-1, keepdims=True))
    return u


@pytest.mark.parametrize("c", [2, 7, 64, 128])
def test_xhat_is_standardised(c):
    rng = np.random.default_rng(c)
    x = rng.standard_normal((5, 3, c)) * 3 + 2
    _, xhat, _, _ = oracle.layer_norm(x, np.ones(c), np.zeros(c), 0.0)
    np.testing.assert_allclose(xhat.mean(axis=-1), 0, atol=1e-13)
    np.testing.assert_allclose((xhat ** 2).mean(axis=-1), 1, atol=1e-13)


def test_shift_and_scale_invariance():
    """Per-token shifts leave the output unchanged for any eps; positive per-token
    scales leave it unchanged when eps = 0."""
    rng = np.random.default_rng(3)
    c = 32
    x = rng.standard_normal((4, 4, c))
    g, b = rng.standard_normal(c), rng.standard_normal(c)
    s = rng.standard_normal((4, 4, 1)) * 10
    a = np.exp(rng.standard_normal((4, 4, 1)))
    y0, _, _, _ = oracle.layer_norm(x, g, b, 1e-3)
    y1, _, _, _ = oracle.layer_norm(x + s, g, b, 1e-3)
    np.testing.assert_allclose(y1, y0, atol=1e-12)
    z0, _, _, _ = oracle.layer_norm(x, g, b, 0.0)
    z1, _, _, _ = oracle.layer_norm(a * x + s, g, b, 0.0)
    np.testing.assert_allclose(z1, z0, atol=1e-12)


@pytest.mark.parametrize("bt", [0, 1])
def test_output_layout_with_selection_weights(bt):
    """Tokens that are a positive multiple of a standardised vector u_t plus an
    offset normalise to u_t exactly (eps = 0), so y_t = gamma*u_t + beta is known
    without the oracle.  Weight rows that each pick one channel (times a distinct
    factor) then fix where every output lands: q/k/v rows in the order q, k, v
    with o = h*d + e, and the bias in [H, A, B] (transposed when bt = 1)."""
    rng = np.random.default_rng(11)
    A, c, H, D = 5, 16, 2, 4
    hd = H * D
    u = standardised(rng, (A, A, c))
    x = np.exp(rng.standard_normal((A, A, 1))) * u + rng.standard_normal((A, A, 1))
    gamma = 1 + 0.5 * rng.standard_normal(c)
    beta = rng.standard_normal(c)
    y = gamma * u + beta
    pick = rng.integers(0, c, size=3 * hd)
    factor = 1.0 + np.arange(3 * hd)
    w = np.zeros((3 * hd, c))
    w[np.arange(3 * hd), pick] = factor
    bpick = rng.integers(0, c, size=H)
    wb = np.zeros((H, c))
    wb[np.arange(H), bpick] = [3.0, -2.0]
    out = fwd(x, gamma, beta, 0.0, w, wb, H, D, bt)
    for which, name in enumerate(("q", "k", "v")):
        for h in range(H):
            for e in range(D):
                o = which * hd + h * D + e
                np.testing.assert_allclose(out[name][:, :, h, e], factor[o] * y[:, :, pick[o]], atol=1e-12)
    for h in range(H):
        tok = wb[h, bpick[h]] * y[:, :, bpick[h]]
        np.testing.assert_allclose(out["bias"][h], tok.T if bt else tok, atol=1e-12)


# ---------------------------------------------------------------- backward

def loss(o, inp):
    s = 0.0
    for n, g in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("bias", "dbias")):
        if o[n] is not None:
            s += float((o[n] * inp[g]).sum())
    return s


def np_inputs(A, B, c, H, D, seed, qkv=True, bias=True):
    t = generate_proj(A, B, c, H, D, dtype=torch.float64, qkv=qkv, bias=bias, seed=seed)
    return {k: (v.double().numpy() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}


@pytest.mark.parametrize("bt,qkv,bias", [(0, True, True), (1, True, True), (0, True, False), (1, False, True)])
def test_gradients_by_central_differences(bt, qkv, bias):
    A = B = 3
    c, H, D = 6, 2, 2
    inp = np_inputs(A, B, c, H, D, seed=5 + bt, qkv=qkv, bias=bias)
    eps = 0.1
    args = lambda p: (p["x"], p["gamma"], p["beta"], eps, p["w_qkv"], p["w_bias"], H, D, bt)
    g = oracle.ln_proj_bwd(*args(inp), inp["dq"], inp["dk"], inp["dv"], inp["dbias"])
    names = [("x", "dx"), ("gamma", "dgamma"), ("beta", "dbeta")]
    if qkv:
        names.append(("w_qkv", "dw_qkv"))
    if bias:
        names.append(("w_bias", "dw_bias"))
    h = 1e-6
    for pname, gname in names:
        base = inp[pname]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = dict(inp), dict(inp)
            bp, bm = base.copy(), base.copy()
            bp[idx] += h
            bm[idx] -= h
            plus[pname], minus[pname] = bp, bm
            fd[idx] = (loss(oracle.ln_proj_fwd(*args(plus)), inp)
                       - loss(oracle.ln_proj_fwd(*args(minus)), inp)) / (2 * h)
        scale = max(1.0, np.abs(fd).max())
        np.testing.assert_allclose(g[gname], fd, rtol=0, atol=1e-7 * scale, err_msg=gname)
    if not qkv:
        assert g["dw_qkv"] is None
    if not bias:
        assert g["dw_bias"] is None


def test_dx_is_orthogonal_to_shift_and_scale():
    """Layer norm ignores a per-token shift (any eps), so each token's dx sums to 0;
    with eps = 0 it ignores a positive per-token scale, so dx is orthogonal to x - mean."""
    inp = np_inputs(4, 4, 24, 2, 4, seed=9)
    for eps in (1e-5, 0.0):
        g = oracle.ln_proj_bwd(inp["x"], inp["gamma"], inp["beta"], eps, inp["w_qkv"], inp["w_bias"], 2, 4, 0,
                               inp["dq"], inp["dk"], inp["dv"], inp["dbias"])
        dx = g["dx"]
        assert np.abs(dx.sum(axis=-1)).max() < 1e-12 * np.abs(dx).max() * 24
        if eps == 0.0:
            cen = inp["x"] - inp["x"].mean(axis=-1, keepdims=True)
            assert np.abs((dx * cen).sum(axis=-1)).max() < 1e-11 * np.abs(dx).max() * np.abs(cen).max() * 24
