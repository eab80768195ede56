"""Pins for the CPU fp64 oracle, independent of the oracle's own code.

Each test fixes part of the oracle against something other than itself:
hand-derived closed forms, invariants of softmax attention, central finite
differences of the oracle's own forward (which checks the backward code), and
torch's fp64 scaled-dot-product attention with autograd (the operator is
standard attention with an additive float mask).  The definition followed is
the exact attention with an additively broadcast pair bias that the MegaFold
pages describe (gist.science technical summary, Methodik section 1).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_n2.json")


def case(R, N, H, D, *, transpose=0, bias=True, mask="mixed", seed=0, bias_std=1.0):
    t = generate(R, N, H, D, dtype=torch.float64, transpose=transpose, bias_std=bias_std,
                 seed=seed, with_bias=bias)
    q, k, v, b, do = (None if t[x] is None else t[x].numpy() for x in ("q", "k", "v", "bias", "dout"))
    m = None
    if mask == "mixed":
        # finite and -inf entries, never a fully masked row
        rng = np.random.default_rng(seed + 1)
        m = rng.standard_normal((R, N)) * 0.5
        m[:, -1] = -np.inf
        if N > 3:
            m[0, 1] = -np.inf
    elif mask == "tail":
        m = np.zeros((R, N))
        m[:, N - max(1, N // 4):] = -np.inf
    return q, k, v, b, m, do


def to_kernel_frame(x, transpose):
    return np.ascontiguousarray(np.swapaxes(x, 0, 1)) if transpose else x


# ---------------------------------------------------------------- worked example

def test_golden_hand_worked_cases():
    data = json.load(open(GOLDEN))
    for c in data["cases"]:
        arr = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
        q, k, v, b, m, do = (arr(c[x]) for x in ("q", "k", "v", "bias", "mask", "dout"))
        o, lse = oracle.fwd(q, k, v, b, m, c["transpose"])
        dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, c["transpose"])
        e = c["expect"]
        for name, got in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            np.testing.assert_allclose(got, np.asarray(e[name]), rtol=0, atol=1e-12, err_msg=c["name"] + ":" + name)
        if b is not None:
            np.testing.assert_allclose(db, np.asarray(e["dbias"]), rtol=0, atol=1e-12)
        else:
            # with no bias input dBias is still the sum of dS over rows
            np.testing.assert_allclose(db, np.asarray(e["dbias"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("transpose", [0, 1])
def test_softmax_rows_sum_to_one(transpose):
    """With v = 1 every output channel equals sum_k P[j,k] = 1."""
    q, k, v, b, m, _ = case(3, 7, 2, 5, transpose=transpose)
    o, _ = oracle.fwd(q, k, np.ones_like(v), b, m, transpose)
    assert np.max(np.abs(o - 1.0)) <= 1e-12


@pytest.mark.parametrize("transpose", [0, 1])
def test_bias_row_shift_invariance(transpose):
    """bias[h,j,:] += c[h,j] leaves O and all gradients unchanged and shifts lse by c."""
    q, k, v, b, m, do = case(3, 6, 2, 4, transpose=transpose)
    c = np.random.default_rng(5).standard_normal(b.shape[:2]) * 3.0
    b2 = b + c[:, :, None]
    o1, l1 = oracle.fwd(q, k, v, b, m, transpose)
    o2, l2 = oracle.fwd(q, k, v, b2, m, transpose)
    g1 = oracle.bwd(q, k, v, b, m, do, transpose)
    g2 = oracle.bwd(q, k, v, b2, m, do, transpose)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    R = m.shape[0]
    np.testing.assert_allclose(l2, l1 + np.broadcast_to(c[None], (R,) + c.shape), rtol=0, atol=1e-12)
    for a, bb in zip(g1, g2):
        np.testing.assert_allclose(bb, a, rtol=0, atol=1e-11)


def _q_zero_reference(v, bias, mask, transpose):
    """O[r,j,h] = sum_k softmax_k(bias[h,j,k] + mask[r,k]) v[r,k,h], a separate direct routine."""
    vk = to_kernel_frame(v, transpose)
    R, N, H, D = vk.shape
    out = np.zeros_like(vk)
    for r in range(R):
        for h in range(H):
            for j in range(N):
                logits = bias[h, j, :] + (mask[r] if mask is not None else 0.0)
                w = np.exp(logits - logits.max())
                w /= w.sum()
                out[r, j, h, :] = w @ vk[r, :, h, :]
    return to_kernel_frame(out, transpose)


@pytest.mark.parametrize("transpose", [0, 1])
def test_q_zero_reduces_to_bias_softmax_mean(transpose):
    q, k, v, b, m, _ = case(4, 6, 3, 4, transpose=transpose)
    o, _ = oracle.fwd(np.zeros_like(q), k, v, b, m, transpose)
    np.testing.assert_allclose(o, _q_zero_reference(v, b, m, transpose), rtol=0, atol=1e-12)


def test_uniform_logits_closed_form():
    """q = 0, bias = 0, last m keys masked: O = mean of unmasked v, lse = log(N - m)."""
    R, N, H, D, mt = 3, 8, 2, 4, 3
    _, k, v, _, _, _ = case(R, N, H, D, mask=None)
    m = np.zeros((R, N))
    m[:, N - mt:] = -np.inf
    o, lse = oracle.fwd(np.zeros_like(k), k, v, np.zeros((H, N, N)), m, 0)
    np.testing.assert_allclose(lse, np.full((R, H, N), math.log(N - mt)), rtol=0, atol=1e-14)
    mean = v[:, : N - mt].mean(axis=1, keepdims=True)
    np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-12)


def test_single_position_closed_form():
    """N = 1: O = v, lse = the single logit, dQ = dK = dBias = 0, dV = dO."""
    R, H, D = 3, 2, 4
    q, k, v, b, _, do = case(R, 1, H, D, mask=None)
    m = np.random.default_rng(2).standard_normal((R, 1))
    o, lse = oracle.fwd(q, k, v, b, m, 0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    s = np.einsum("rphc,rphc->rhp", q, k) / math.sqrt(D) + b[None, :, 0, :] + m[:, None, :]
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-14)
    dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, 0)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(db == 0)
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


def test_single_unmasked_key():
    """Only key k* unmasked: O = v[k*], and gradients wrt q, k and bias vanish."""
    R, N, H, D, ks = 2, 6, 2, 3, 4
    q, k, v, b, _, do = case(R, N, H, D, mask=None)
    m = np.full((R, N), -np.inf)
    m[:, ks] = 0.0
    o, lse = oracle.fwd(q, k, v, b, m, 0)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, ks:ks + 1], o.shape), rtol=0, atol=1e-14)
    dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, 0)
    assert np.max(np.abs(dq)) == 0 and np.max(np.abs(dk)) == 0 and np.max(np.abs(db)) == 0
    expect_dv = np.zeros_like(v)
    expect_dv[:, ks] = do.sum(axis=1)
    np.testing.assert_allclose(dv, expect_dv, rtol=0, atol=1e-13)


def test_fully_masked_row_convention():
    """A row whose keys are all masked: O = 0, lse = -inf, no gradient contribution."""
    R, N, H, D = 3, 5, 2, 4
    q, k, v, b, _, do = case(R, N, H, D, mask=None)
    m = np.zeros((R, N))
    m[1, :] = -np.inf
    o, lse = oracle.fwd(q, k, v, b, m, 0)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, 0)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)
    # dBias equals the sum over the other rows only
    keep = [0, 2]
    _, _, _, db_keep = oracle.bwd(q, k, v, b, m, do, 0, rows=keep)
    np.testing.assert_array_equal(db, db_keep)


@pytest.mark.parametrize("transpose", [0, 1])
def test_gradient_sum_identities(transpose):
    """Each dS row sums to zero, so sum_k dBias = 0; P is row-stochastic, so sum_k dV = sum_j dO."""
    q, k, v, b, m, do = case(3, 7, 2, 4, transpose=transpose)
    dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, transpose)
    assert np.max(np.abs(db.sum(axis=2))) <= 1e-12
    ax = 0 if transpose else 1
    np.testing.assert_allclose(dv.sum(axis=ax), do.sum(axis=ax), rtol=0, atol=1e-12)
    # sum over keys of dK is dQ-like: sum_k dS[j,k] = 0 gives sum_k dK = 0 as well
    assert np.max(np.abs(dk.sum(axis=ax))) <= 1e-12


def test_delta_identity():
    """sum_k P dP = sum_c dO * O (the identity a fused backward uses), via the oracle's O and
    a direct evaluation of P and dP from their definitions."""
    R, N, H, D = 2, 6, 2, 4
    q, k, v, b, m, do = case(R, N, H, D)
    o, lse = oracle.fwd(q, k, v, b, m, 0)
    s = np.einsum("rjhc,rkhc->rhjk", q, k) / math.sqrt(D) + b[None] + m[:, None, None, :]
    p = np.exp(s - lse[..., None])
    dp = np.einsum("rjhc,rkhc->rhjk", do, v)
    lhs = (p * dp).sum(-1)
    rhs = np.einsum("rjhc,rjhc->rhj", do, o)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


def test_transpose_is_permutation_exactly():
    """F(transpose=1, X) = T(F(transpose=0, T(X))) bit for bit (same arithmetic, other addressing)."""
    q, k, v, b, m, do = case(5, 5, 2, 4, transpose=0)
    T = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
    o0, l0 = oracle.fwd(q, k, v, b, m, 0)
    o1, l1 = oracle.fwd(T(q), T(k), T(v), b, m, 1)
    np.testing.assert_array_equal(T(o1), o0)
    np.testing.assert_array_equal(l1, l0)
    g0 = oracle.bwd(q, k, v, b, m, do, 0)
    g1 = oracle.bwd(T(q), T(k), T(v), b, m, T(do), 1)
    for a, c in zip(g0[:3], g1[:3]):
        np.testing.assert_array_equal(T(c), a)
    np.testing.assert_array_equal(g1[3], g0[3])


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("transpose", [0, 1])
def test_central_finite_differences(transpose):
    """All four gradients equal central differences of L = sum(O * dO) (fp64, eps = 1e-6)."""
    R, N, H, D = 2, 4, 2, 3
    q, k, v, b, m, do = case(R, N, H, D, transpose=transpose, seed=3)
    m[1, 0] = 0.7   # a finite, nonzero mask entry too
    dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, transpose)
    eps = 1e-6

    def loss(qq, kk, vv, bb):
        o, _ = oracle.fwd(qq, kk, vv, bb, m, transpose)
        return float(np.sum(o * do))

    inputs = [q, k, v, b]
    grads = [dq, dk, dv, db]
    for idx, (x, g) in enumerate(zip(inputs, grads)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp = x.copy(); xp[pos] += eps
            xm = x.copy(); xm[pos] -= eps
            args_p = list(inputs); args_p[idx] = xp
            args_m = list(inputs); args_m[idx] = xm
            num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err <= 1e-6, (idx, err)


# ---------------------------------------------------------------- library cross-check

@pytest.mark.parametrize("transpose", [0, 1])
@pytest.mark.parametrize("shape", [(3, 9, 2, 8), (2, 17, 3, 32)])
def test_against_torch_sdpa_fp64(transpose, shape):
    """Forward and all gradients equal torch's math SDPA in fp64 with a float attn_mask
    bias[None] + mask[:, None, None, :]; dBias = sum over rows of d(attn_mask)."""
    R, N, H, D = shape
    q, k, v, b, m, do = case(R, N, H, D, transpose=transpose, seed=7, bias_std=math.sqrt(2))
    o, lse = oracle.fwd(q, k, v, b, m, transpose)
    dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, transpose)

    def kf(x):  # physical -> [R, H, N, D]
        return torch.from_numpy(to_kernel_frame(x, transpose)).permute(0, 2, 1, 3).contiguous()

    tq, tk, tv = (kf(x).requires_grad_(True) for x in (q, k, v))
    tb = torch.from_numpy(b).requires_grad_(True)
    am = tb[None] + torch.from_numpy(m)[:, None, None, :]
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am)
    to.backward(kf(do))
    back = lambda t: to_kernel_frame(t.detach().permute(0, 2, 1, 3).numpy(), transpose)
    np.testing.assert_allclose(o, back(to), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, back(tq.grad), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, back(tk.grad), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, back(tv.grad), rtol=0, atol=1e-11)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=0, atol=1e-11)
    # lse against torch.logsumexp of the logits formed with torch ops
    logits = (tq.detach() @ tk.detach().transpose(-1, -2)) / math.sqrt(D) + am.detach()
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- row subsets, threads

def test_row_subset_matches_full_run():
    """Rows computed alone equal the full run bit for bit; with dO = 0 outside the subset the
    full dBias equals the subset's dBias bit for bit (the basis of sampled large-size parity)."""
    R, N, H, D = 6, 7, 2, 4
    q, k, v, b, m, do = case(R, N, H, D)
    rows = [1, 4, 5]
    o, lse = oracle.fwd(q, k, v, b, m, 0)
    os_, ls = oracle.fwd(q, k, v, b, m, 0, rows=rows)
    np.testing.assert_array_equal(os_[rows], o[rows])
    np.testing.assert_array_equal(ls[rows], lse[rows])
    assert np.all(np.isnan(os_[[0, 2, 3]]))
    do_s = np.zeros_like(do)
    do_s[rows] = do[rows]
    full = oracle.bwd(q, k, v, b, m, do_s, 0)
    sub = oracle.bwd(q, k, v, b, m, do, 0, rows=rows)
    for a, c in zip(full[:3], sub[:3]):
        np.testing.assert_array_equal(c[rows], a[rows])
    np.testing.assert_array_equal(sub[3], full[3])


def test_thread_count_does_not_change_results():
    q, k, v, b, m, do = case(5, 12, 3, 8)
    prev = oracle.set_threads(0)
    try:
        oracle.set_threads(1)
        g1 = oracle.bwd(q, k, v, b, m, do, 0)
        oracle.set_threads(4)
        g4 = oracle.bwd(q, k, v, b, m, do, 0)
    finally:
        oracle.set_threads(prev)
    for a, c in zip(g1, g4):
        np.testing.assert_array_equal(a, c)
