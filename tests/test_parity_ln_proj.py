"""GPU parity of the fused layer norm + projections against the fp64 oracle, on the
same seeded inputs, through the C ABI.

Tolerances, per output element, from the arithmetic (S = sum_c |y_c| |w_c| with
y the exact layer-norm output and w the weight row):
  bf16: the kernel rounds y to bf16 (relative error <= 2^-9 per term, so the sum
        moves by <= 2^-9 S), accumulates in fp32 and rounds the result to bf16
        (<= 2^-9 of |out| <= 2^-9 S): |err| <= 2^-8 S, with 1/64 of headroom for
        the fp32 statistics and sums.
  fp32: fp32 statistics and a C-term fp32 sum: |err| <= (C + 8) 2^-24 S.
  mean: within 1e-6 * max|x| + 1e-6; rstd: relative 1e-4 (fp32 two-pass variance
        and a hardware reciprocal square root).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import PROJ_WORKLOADS, generate_proj, generate_proj_workload

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[ln_proj] {msg}", flush=True)


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def run_gpu(inp, bias_transpose):
    import af3_attention_amd as ea
    dev = torch.device("cuda:0")
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = ea.ln_proj_fwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], heads=inp["heads"],
                         head_dim=inp["head_dim"], bias_transpose=bias_transpose, eps=inp["eps"])
    torch.cuda.synchronize()
    return out


def check(inp, bias_transpose, mode, ia=None, ib=None):
    """Compares every output, or (with index sets ia, ib of equal length) the outputs
    of the token sub-grid ia x ib; layer norm and projections act token by token,
    so the oracle on the sub-grid gives exactly those outputs."""
    H, D = inp["heads"], inp["head_dim"]
    got = run_gpu(inp, bias_transpose)
    for n in ("q", "k", "v", "bias", "mean", "rstd"):
        if got[n] is not None:
            assert bool(torch.isfinite(got[n]).all()), f"{n}: non-finite values"
    x = inp["x"]
    if ia is not None:
        x = x[ia][:, ib]
        sub = lambda t: t[ia][:, ib]
        got = {"q": None, "k": None, "v": None, "bias": None,
               **{n: sub(got[n]) for n in ("q", "k", "v") if got[n] is not None},
               "mean": sub(got["mean"].view(inp["x"].shape[:2])), "rstd": sub(got["rstd"].view(inp["x"].shape[:2])),
               "bias": None if got["bias"] is None else (
                   got["bias"][:, ib][:, :, ia] if bias_transpose else got["bias"][:, ia][:, :, ib])}
    x, gamma, beta = f64(x), f64(inp["gamma"]), f64(inp["beta"])
    wq, wb = f64(inp["w_qkv"]), f64(inp["w_bias"])
    ref = oracle.ln_proj_fwd(x, gamma, beta, inp["eps"], wq, wb, H, D, bias_transpose)
    A, B, C = x.shape
    y, _, _, _ = oracle.layer_norm(x, gamma, beta, inp["eps"])
    ay = np.abs(y).reshape(A * B, C)
    factor = 2.0 ** -8 * (1 + 2.0 ** -6) if mode == "bf16" else (C + 8) * 2.0 ** -24
    errs = {}
    if wq is not None:
        S = (ay @ np.abs(wq).T).reshape(A, B, 3, H, D)
        for i, n in enumerate(("q", "k", "v")):
            g, r = f64(got[n]), ref[n]
            tol = factor * S[:, :, i] + 1e-7
            err = np.abs(g - r)
            errs[n] = float((err / tol).max())
            assert np.all(np.isfinite(g)), n
            assert np.all(err <= tol), f"{n}: worst err/tol {errs[n]:.3f} at {np.unravel_index(np.argmax(err / tol), err.shape)}"
    else:
        assert got["q"] is None
    if wb is not None:
        Sb = np.moveaxis((ay @ np.abs(wb).T).reshape(A, B, H), -1, 0)
        if bias_transpose:
            Sb = Sb.transpose(0, 2, 1)
        g, r = f64(got["bias"]), ref["bias"]
        tol = factor * Sb + 1e-7
        err = np.abs(g - r)
        errs["bias"] = float((err / tol).max())
        assert np.all(err <= tol), f"bias: worst err/tol {errs['bias']:.3f}"
    else:
        assert got["bias"] is None
    gm, gr = f64(got["mean"]).reshape(A, B), f64(got["rstd"]).reshape(A, B)
    assert np.abs(gm - ref["mean"]).max() <= 1e-6 * np.abs(x).max() + 1e-6
    assert np.abs(gr / ref["rstd"] - 1).max() <= 1e-4
    print(errs, flush=True)
    return errs


def dtype_of(mode):
    return torch.float32 if mode == "fp32" else torch.bfloat16


# ---------------------------------------------------------------- every element

def test_fp32_workload():
    w = PROJ_WORKLOADS["pair_proj_fp32_n64"]
    banner(w.name)
    check(generate_proj_workload(w), 0, "fp32")


@pytest.mark.parametrize("bt", [0, 1])
@pytest.mark.parametrize("N", [50, 64, 97])
def test_bf16_pair_c128(N, bt):
    """MFMA kernel, the pair-tensor shape (C=128, H=4, d=32) with a ragged last tile."""
    banner(f"bf16 pair N={N} C=128 bt={bt}")
    check(generate_proj(N, N, 128, 4, 32, dtype=torch.bfloat16, seed=N + bt), bt, "bf16")


@pytest.mark.parametrize("A,B,C,H,D,qkv,bias,bt", [
    (37, 45, 64, 8, 8, True, False, 0),     # MSA-like: q, k, v only
    (33, 33, 64, 4, 32, False, True, 0),    # bias only, one partly used weight tile
    (33, 33, 64, 4, 32, False, True, 1),
    (40, 40, 32, 1, 8, True, True, 0),      # n_qkv = 24: q/k/v and bias share a weight tile
    (40, 40, 32, 1, 8, True, True, 1),
    (29, 29, 128, 2, 64, True, True, 1),
    (1, 1, 128, 4, 32, True, True, 0),      # a single token
])
def test_bf16_shapes(A, B, C, H, D, qkv, bias, bt):
    banner(f"bf16 A={A} B={B} C={C} H={H} D={D} qkv={qkv} bias={bias} bt={bt}")
    check(generate_proj(A, B, C, H, D, dtype=torch.bfloat16, qkv=qkv, bias=bias, seed=A * 3 + C), bt, "bf16")


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
@pytest.mark.parametrize("A,C,H,D,bt", [(20, 96, 2, 16, 1), (9, 256, 4, 32, 0), (12, 40, 3, 8, 1)])
def test_vector_kernel_shapes(A, C, H, D, bt, mode):
    """Channel counts outside the MFMA kernel run the vector kernel (fp32 always does)."""
    banner(f"{mode} vector A={A} C={C} H={H} D={D} bt={bt}")
    check(generate_proj(A, A, C, H, D, dtype=dtype_of(mode), seed=C + A), bt, mode)


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_constant_tokens_give_beta(mode):
    """A token whose channels are all equal has zero variance: xhat = 0 and y = beta,
    so every output is beta projected (eps keeps rstd finite)."""
    banner(f"{mode} constant tokens")
    inp = generate_proj(16, 16, 128, 4, 32, dtype=dtype_of(mode), seed=3)
    x = inp["x"].clone()
    x[3, :, :] = 2.5
    x[:, 7, :] = -1.0
    inp["x"] = x
    check(inp, 0, mode)


# ---------------------------------------------------------------- full workload sizes

def sample_axis(n, k, seed):
    """k sorted distinct indices of range(n) that include both ends."""
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n - 1), size=k - 2, replace=False)
    return torch.as_tensor(np.sort(np.concatenate([[0, n - 1], mid])), dtype=torch.long)


@pytest.mark.parametrize("name", ["pair_proj_bf16_n384", "pair_proj_end_bf16_n768", "msa_proj_bf16_s512_n384"])
def test_bf16_workloads_sampled(name):
    """Full workload sizes in the launch configuration the benchmark times; every
    output is checked finite and a 96 x 96 token sub-grid against the oracle."""
    w = PROJ_WORKLOADS[name]
    banner(w.name)
    k = 96
    check(generate_proj_workload(w), w.bias_transpose, "bf16", sample_axis(w.a, k, 1), sample_axis(w.b, k, 2))
