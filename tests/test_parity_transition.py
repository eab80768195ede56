"""GPU parity of the fused SwiGLU transition against the fp64 oracle, on the same
seeded inputs, through the C ABI.

Forward tolerance per output element, from the arithmetic (bf16 has 8
significant bits, so each rounding moves a value by at most 2^-8 of it):
  y is rounded to bf16, so a and b move by at most Ea = 2^-8 sum_c |y||w_a| and
  Eb = 2^-8 sum_c |y||w_b|; h = silu(a) b then moves by at most
  Eh = |silu'(a)| Ea |b| + |silu(a)| Eb (first order) plus its own rounding to bf16,
  2^-8 |h|; out = sum_j h_j w_out[c, j] moves by sum_j Eh_j |w_out[c, j]| and by
  its final rounding 2^-8 |out|.  The test allows 1.25x that bound (second-order
  terms, the fp32 sums and the hardware exp / reciprocal) plus 1e-6.  The bound
  sums worst cases over n*C terms, so the test also requires max|err| <= 1e-2
  max|ref|: the output's own rounding is 2^-8 (0.4 %) and the upstream rounding
  errors, independent across the n*C terms, add a few tenths of a percent.
mean: within 1e-6 max|x| + 1e-6; rstd: relative 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import TRANSITION_WORKLOADS, generate_transition, generate_transition_workload

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def banner(msg):
    print(f"\n[transition] {msg}", flush=True)


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def gpu_fwd(inp):
    import af3_attention_amd as ea
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = ea.transition_fwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], eps=inp["eps"])
    torch.cuda.synchronize()
    return out


def fwd_bound(x, gamma, beta, eps, wa, wb, wo):
    """Per-element forward error bound (see the module docstring)."""
    A, B, C = x.shape
    y, _, _, _ = oracle.layer_norm(x, gamma, beta, eps)
    y2 = y.reshape(-1, C)
    a, b = y2 @ wa.T, y2 @ wb.T
    h = oracle.silu(a) * b
    Ea = U * (np.abs(y2) @ np.abs(wa).T)
    Eb = U * (np.abs(y2) @ np.abs(wb).T)
    Eh = np.abs(oracle.silu_grad(a)) * Ea * np.abs(b) + np.abs(oracle.silu(a)) * Eb + U * np.abs(h)
    out = h @ wo.T
    return (1.25 * (Eh @ np.abs(wo).T + U * np.abs(out)) + 1e-6).reshape(A, B, C)


def check_fwd(inp, ia=None, ib=None):
    got = gpu_fwd(inp)
    assert bool(torch.isfinite(got["out"]).all())
    x = inp["x"]
    o, mean, rstd = got["out"], got["mean"].view(x.shape[:2]), got["rstd"].view(x.shape[:2])
    if ia is not None:
        x, o, mean, rstd = x[ia][:, ib], o[ia][:, ib], mean[ia][:, ib], rstd[ia][:, ib]
    args = [f64(x), f64(inp["gamma"]), f64(inp["beta"]), inp["eps"], f64(inp["w_a"]), f64(inp["w_b"]),
            f64(inp["w_out"])]
    ref = oracle.transition_fwd(*args)
    tol = fwd_bound(*args)
    err = np.abs(f64(o) - ref["out"])
    worst = float((err / tol).max())
    rel = float(err.max() / np.abs(ref["out"]).max())
    print({"out err/tol": worst, "max err / max ref": rel}, flush=True)
    assert np.all(err <= tol), f"out: worst err/tol {worst:.3f}"
    assert rel <= 1e-2, f"out: max err / max|ref| = {rel:.2e}"
    assert np.abs(f64(mean) - ref["mean"]).max() <= 1e-6 * np.abs(args[0]).max() + 1e-6
    assert np.abs(f64(rstd) / ref["rstd"] - 1).max() <= 1e-4


@pytest.mark.parametrize("A,B,C,n", [(16, 16, 128, 4), (7, 9, 128, 4), (33, 20, 64, 4), (5, 5, 128, 1),
                                     (12, 11, 64, 2), (1, 1, 128, 4), (40, 41, 128, 4)])
def test_fwd_shapes(A, B, C, n):
    """Ragged tiles and passes (token counts not multiples of 32 or 256), both channel
    counts, expansions 1, 2 and 4, a single token."""
    banner(f"fwd A={A} B={B} C={C} n={n}")
    check_fwd(generate_transition(A, B, C, n, dtype=torch.bfloat16, seed=A * 5 + n))


def test_fwd_constant_tokens():
    """Tokens with equal channels normalise to y = beta (zero variance)."""
    banner("fwd constant tokens")
    inp = generate_transition(20, 20, 128, 4, dtype=torch.bfloat16, seed=8)
    x = inp["x"].clone()
    x[2] = 1.5
    x[:, 11] = -3.0
    inp["x"] = x
    check_fwd(inp)


def sample_axis(n, k, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n - 1), size=k - 2, replace=False)
    return torch.as_tensor(np.sort(np.concatenate([[0, n - 1], mid])), dtype=torch.long)


@pytest.mark.parametrize("name", ["pair_transition_bf16_n384", "msa_transition_bf16_s512_n384"])
def test_fwd_workloads_sampled(name):
    """Full sizes in the benchmark's launch configuration; every output finite, a
    48 x 48 token sub-grid against the oracle."""
    w = TRANSITION_WORKLOADS[name]
    banner("fwd " + name)
    check_fwd(generate_transition_workload(w), sample_axis(w.a, 48, 1), sample_axis(w.b, 48, 2))


def test_fwd_unsupported_shapes_fail_loudly():
    import af3_attention_amd as ea
    inp = generate_transition(4, 4, 96, 2, dtype=torch.bfloat16, seed=0)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    with pytest.raises(ea.EvoAttnError, match="channels"):
        ea.transition_fwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"])
    f = generate_transition(4, 4, 64, 2, dtype=torch.float32, seed=0)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in f.items()}
    with pytest.raises(ea.EvoAttnError, match="bf16"):
        ea.transition_fwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"])


# ================================================================ backward
#
# Every matrix-core operand of the backward (y, xhat, dout, da, db, h) is bf16,
# i.e. rounded by at most 2^-9 of itself (round to nearest, 8 significant bits),
# and each result sums n*C or T such terms in fp32.  The backward rounds x-hat
# twice where the forward rounds it once: the dx kernel forms y from the
# bf16-rounded x-hat it hands to the weight-gradient kernel (y = gamma bf16(xhat)
# + beta, rounded again), so y, a and b carry two roundings, at most about 2^-8
# relative together, while the layer-norm part of dx uses the fp32 x-hat.
# Independent roundings of that size give each gradient a relative error of a few
# tenths of a percent of its max norm (the forward's is 0.3-0.5 %, the measured
# backward errors 0.3-0.5 %); dx also carries its own final rounding.  The test
# requires max|err| <= 2e-2 max|ref| for dx and every weight gradient, and
# bit-identical results from two calls.

BWD_REL = 2e-2


def gpu_bwd(inp, reps=2):
    import af3_attention_amd as ea
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    fw = ea.transition_fwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], eps=inp["eps"])
    outs = [ea.transition_bwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], fw["mean"],
                              fw["rstd"], g["dout"]) for _ in range(reps)]
    torch.cuda.synchronize()
    return outs


def check_bwd(inp, ia=None, ib=None):
    got, again = gpu_bwd(inp)
    for n in got:
        assert torch.equal(got[n], again[n]), f"{n}: two calls differ"
        assert bool(torch.isfinite(got[n]).all()), f"{n}: non-finite"
    sub = inp
    dx = got["dx"]
    if ia is not None:
        keep = torch.zeros(inp["x"].shape[:2], dtype=torch.bool)
        keep[ia[:, None], ib[None, :]] = True
        assert bool((dx.cpu()[~keep] == 0).all()), "dx must vanish where dout is zero"
        dx = dx[ia][:, ib]
        sub = dict(inp)
        sub["x"] = inp["x"][ia][:, ib]
        sub["dout"] = inp["dout"][ia][:, ib]
    ref = oracle.transition_bwd(f64(sub["x"]), f64(sub["gamma"]), f64(sub["beta"]), sub["eps"], f64(sub["w_a"]),
                                f64(sub["w_b"]), f64(sub["w_out"]), f64(sub["dout"]))
    errs = {}
    for n in ("dx", "dgamma", "dbeta", "dw_a", "dw_b", "dw_out"):
        g = f64(dx) if n == "dx" else f64(got[n])
        e = float(np.abs(g - ref[n]).max() / np.abs(ref[n]).max())
        errs[n] = e
    print("bwd", errs, flush=True)
    for n, e in errs.items():
        assert e <= BWD_REL, f"{n}: max err / max|ref| = {e:.2e}"


@pytest.mark.parametrize("A,B,C,n", [(16, 16, 128, 4), (7, 9, 128, 4), (33, 20, 64, 4), (5, 5, 128, 1),
                                     (12, 11, 64, 2), (1, 1, 128, 4), (40, 41, 128, 4), (70, 70, 64, 4),
                                     (72, 72, 128, 4), (100, 100, 128, 4), (50, 90, 64, 4)])
def test_bwd_shapes(A, B, C, n):
    """Ragged tiles and token ranges; the weight-gradient kernel's per-range chunk
    counts cover 1, 2, 3 and 5 (with a shorter last range and a partial last chunk),
    besides the full-size cases below."""
    banner(f"bwd A={A} B={B} C={C} n={n}")
    check_bwd(generate_transition(A, B, C, n, dtype=torch.bfloat16, seed=A * 7 + n))


@pytest.mark.parametrize("A,B,C", [(7, 9, 128), (33, 20, 64)])
def test_bwd_ignores_workspace_contents(A, B, C):
    """The workspace (partial sums, and the bf16 xhat rows the dx kernel hands to
    the weight-gradient kernel, in whole 256-token passes) may hold anything on
    entry: a workspace of NaN bytes gives the same bits as a zeroed one."""
    import af3_attention_amd as ea
    banner(f"bwd workspace contents A={A} B={B} C={C}")
    inp = generate_transition(A, B, C, 4, dtype=torch.bfloat16, seed=A + B)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    fw = ea.transition_fwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], eps=inp["eps"])
    nbytes = ea.transition_bwd_workspace_bytes(A, B, C, 4)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        outs.append(ea.transition_bwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], fw["mean"],
                                      fw["rstd"], g["dout"], workspace=ws))
    torch.cuda.synchronize()
    for n in outs[0]:
        assert bool(torch.isfinite(outs[1][n]).all()), f"{n}: non-finite with a NaN-filled workspace"
        assert torch.equal(outs[0][n], outs[1][n]), f"{n}: depends on the workspace contents"


@pytest.mark.parametrize("name", ["pair_transition_bf16_n384", "msa_transition_bf16_s512_n384"])
def test_bwd_workloads_sampled(name):
    """Full sizes in the benchmark's launch configuration with dout zero outside a
    40 x 40 token sub-grid: the weight gradients then equal the sub-grid's
    exactly, dx matches on it and vanishes elsewhere."""
    w = TRANSITION_WORKLOADS[name]
    banner("bwd " + name)
    inp = generate_transition_workload(w)
    ia, ib = sample_axis(w.a, 40, 3), sample_axis(w.b, 40, 4)
    keep = torch.zeros((w.a, w.b), dtype=torch.bool)
    keep[ia[:, None], ib[None, :]] = True
    inp["dout"] = inp["dout"] * keep[:, :, None].to(inp["dout"].dtype)
    check_bwd(inp, ia, ib)


def test_autograd_matches_entry_points():
    import af3_attention_amd as ea
    banner("transition autograd")
    inp = generate_transition(20, 24, 128, 4, dtype=torch.bfloat16, seed=11)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    leaves = {n: g[n].clone().requires_grad_(True) for n in ("x", "gamma", "beta", "w_a", "w_b", "w_out")}
    out = ea.transition(leaves["x"], leaves["gamma"], leaves["beta"], leaves["w_a"], leaves["w_b"], leaves["w_out"])
    (out.float() * g["dout"].float()).sum().backward()
    fw = ea.transition_fwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"])
    ref = ea.transition_bwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], fw["mean"], fw["rstd"],
                            g["dout"])
    torch.cuda.synchronize()
    assert torch.equal(out, fw["out"])
    assert torch.equal(leaves["x"].grad, ref["dx"])
    assert torch.equal(leaves["gamma"].grad, ref["dgamma"]) and torch.equal(leaves["beta"].grad, ref["dbeta"])
    for n in ("w_a", "w_b", "w_out"):
        assert torch.equal(leaves[n].grad, ref["d" + n].to(torch.bfloat16)), n
