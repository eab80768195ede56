"""Pins for the fp64 oracle of the SwiGLU transition (EvoFusion's gated group),
independent of the oracle's own code: a hand-derived example, closed forms and
identities of silu, linearity, and central finite differences of every gradient.
The pages (MegaFold, gist.science technical summary, Methodik section 3
"EvoFusion") name SwiGLU among the fused operators but print no formula."""
import numpy as np
import pytest
import torch

import oracle
from workloads import generate_transition

SIG1 = 0.7310585786300049  # 1 / (1 + e^-1)


def test_two_channel_example_by_hand():
    """x = [3, 1] normalises to y = [1, -1] (eps = 0, gamma = 1, beta = 0).  With
    w_a = I, a = [1, -1]; w_b = [[2, 0], [1, 1]] gives b = [2, 0]; so
    h = [silu(1) * 2, silu(-1) * 0] = [2 sigma(1), 0], and w_out = [[1, 1], [0.5, -1]]
    gives out = [2 sigma(1), sigma(1)].  (Gating b instead of a would give
    [silu(2), 0]-based values.)"""
    out = oracle.transition_fwd(np.array([[[3.0, 1.0]]]), np.ones(2), np.zeros(2), 0.0,
                                np.eye(2), np.array([[2.0, 0.0], [1.0, 1.0]]), np.array([[1.0, 1.0], [0.5, -1.0]]))
    np.testing.assert_allclose(out["out"].ravel(), [2 * SIG1, SIG1], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out["mean"].ravel(), [2.0], atol=1e-15)
    np.testing.assert_allclose(out["rstd"].ravel(), [1.0], atol=1e-15)


def test_silu_closed_forms_and_identities():
    assert oracle.silu(np.array(0.0)) == 0.0
    assert oracle.silu_grad(np.array(0.0)) == 0.5
    np.testing.assert_allclose(oracle.silu(np.array(1.0)), SIG1, atol=1e-16)
    x = np.linspace(-30, 30, 601)
    # silu(x) - silu(-x) = x and silu'(x) + silu'(-x) = 1 for every x
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, atol=1e-12)
    np.testing.assert_allclose(oracle.silu_grad(x) + oracle.silu_grad(-x), 1.0, atol=1e-12)
    # tails: silu(x) -> x for large x, -> 0 for very negative x
    assert abs(oracle.silu(np.array(40.0)) - 40.0) < 1e-12
    assert abs(oracle.silu(np.array(-40.0))) < 1e-15
    # derivative by central differences
    h = 1e-6
    np.testing.assert_allclose((oracle.silu(x + h) - oracle.silu(x - h)) / (2 * h), oracle.silu_grad(x), atol=1e-8)


def np_inputs(A, B, C, n, seed):
    t = generate_transition(A, B, C, n, dtype=torch.float64, seed=seed)
    return {k: (v.double().numpy() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}


def test_linear_in_w_b_and_w_out():
    p = np_inputs(3, 4, 16, 2, seed=2)
    f = lambda **kw: oracle.transition_fwd(p["x"], p["gamma"], p["beta"], p["eps"], kw.get("wa", p["w_a"]),
                                           kw.get("wb", p["w_b"]), kw.get("wo", p["w_out"]))["out"]
    base = f()
    np.testing.assert_allclose(f(wb=2.5 * p["w_b"]), 2.5 * base, atol=1e-12)
    w2 = np.random.default_rng(0).standard_normal(p["w_out"].shape)
    np.testing.assert_allclose(f(wo=p["w_out"] + w2), base + f(wo=w2), atol=1e-12)
    # and not linear in w_a (the gate)
    assert np.abs(f(wa=2 * p["w_a"]) - 2 * base).max() > 1e-3


def loss(p, eps):
    out = oracle.transition_fwd(p["x"], p["gamma"], p["beta"], eps, p["w_a"], p["w_b"], p["w_out"])["out"]
    return float((out * p["dout"]).sum())


@pytest.mark.parametrize("seed", [3, 4])
def test_gradients_by_central_differences(seed):
    p = np_inputs(2, 3, 6, 2, seed=seed)
    eps = 0.05
    g = oracle.transition_bwd(p["x"], p["gamma"], p["beta"], eps, p["w_a"], p["w_b"], p["w_out"], p["dout"])
    h = 1e-6
    for pname, gname in (("x", "dx"), ("gamma", "dgamma"), ("beta", "dbeta"), ("w_a", "dw_a"), ("w_b", "dw_b"),
                         ("w_out", "dw_out")):
        base = p[pname]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = dict(p), dict(p)
            bp, bm = base.copy(), base.copy()
            bp[idx] += h
            bm[idx] -= h
            plus[pname], minus[pname] = bp, bm
            fd[idx] = (loss(plus, eps) - loss(minus, eps)) / (2 * h)
        scale = max(1.0, np.abs(fd).max())
        np.testing.assert_allclose(g[gname], fd, rtol=0, atol=1e-7 * scale, err_msg=gname)


def test_dx_sums_to_zero_per_token():
    p = np_inputs(4, 4, 32, 4, seed=6)
    g = oracle.transition_bwd(p["x"], p["gamma"], p["beta"], 1e-5, p["w_a"], p["w_b"], p["w_out"], p["dout"])
    assert np.abs(g["dx"].sum(axis=-1)).max() < 1e-12 * np.abs(g["dx"]).max() * 32
