"""GPU parity of the fused layer norm + projections against the fp64 oracle, on the
same seeded inputs, through the C ABI.

Tolerances, per output element, from the arithmetic (S = sum_c |y_c| |w_c| with
y the exact layer-norm output and w the weight row):
  bf16: the kernel rounds y to bf16 (8 significant bits: relative error <= 2^-8
        per term, so the sum moves by <= 2^-8 S), accumulates in fp32 and rounds
        the result to bf16 (<= 2^-8 of |out| <= 2^-8 S): |err| <= 2^-7 S, with
        1/64 of headroom for the fp32 statistics and sums.
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
    factor = 2.0 ** -7 * (1 + 2.0 ** -6) if mode == "bf16" else (C + 8) * 2.0 ** -24
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


# ================================================================ backward
#
# dx, per element (bf16): the kernel's dy is an fp32 sum of exact bf16 products,
# except the pair-bias heads, whose fp32 upstream gradient is rounded to bf16
# (2^-8 relative); the fp32 sum over n_out terms adds at most n_out 2^-24 of
# the absolute terms.  With E_t the largest such dy error of token t, the
# layer-norm backward moves dx by at most delta = rstd_t max|gamma| E_t (2 + |xhat|)
# (mean|xhat| <= 1), and the final rounding to bf16 by 2^-8 |dx|; with 2x
# headroom on the rounding and 20% on delta:
#   |dx - ref| <= 2^-7 |ref| + 1.2 delta + 1e-6.
# fp32: within 1e-5 of each token's largest |dx|.
# dW, dgamma, dbeta are sums over all tokens of terms with xhat rounded to bf16:
# independent rounding errors of relative size <= 2^-8 (standard deviation
# 2^-8/sqrt(3)) give each sum a relative error near 2.3e-3, so the check is
# max|err| <= 1e-2 max|ref| (bf16; ~4x headroom) and 1e-5 (fp32).

BF16_RED_REL = 1e-2
FP32_REL = 1e-5


def bwd_inputs_gpu(inp):
    dev = torch.device("cuda:0")
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_gpu_bwd(inp, bias_transpose, reps=1):
    import af3_attention_amd as ea
    g = bwd_inputs_gpu(inp)
    H, D = inp["heads"], inp["head_dim"]
    fw = ea.ln_proj_fwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], heads=H, head_dim=D,
                        bias_transpose=bias_transpose, eps=inp["eps"])
    outs = []
    for _ in range(reps):
        outs.append(ea.ln_proj_bwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], fw["mean"], fw["rstd"],
                                   g["dq"], g["dk"], g["dv"], g["dbias"], heads=H, head_dim=D,
                                   bias_transpose=bias_transpose))
    torch.cuda.synchronize()
    return outs


def upstream_by_token(inp, bias_transpose):
    """G [T, n_out] in fp64 (dq | dk | dv | bias heads), the kernel's view of the upstream gradients."""
    A, B, C = inp["x"].shape
    H, D = inp["heads"], inp["head_dim"]
    cols = []
    if inp["w_qkv"] is not None:
        cols += [f64(inp[n]).reshape(A * B, H * D) for n in ("dq", "dk", "dv")]
    if inp["w_bias"] is not None:
        db = f64(inp["dbias"])
        db = db.transpose(0, 2, 1) if bias_transpose else db
        cols.append(np.moveaxis(db, 0, -1).reshape(A * B, H))
    return np.concatenate(cols, axis=1)


def check_bwd(inp, bias_transpose, mode, ia=None, ib=None):
    """Compares dx (every token, or the sub-grid ia x ib) and the token reductions.
    With a sub-grid, the upstream gradients must be zero outside it: then the
    reductions are exactly the sub-grid's and dx is zero elsewhere."""
    H, D = inp["heads"], inp["head_dim"]
    got, again = run_gpu_bwd(inp, bias_transpose, reps=2)
    for n in ("dgamma", "dbeta", "dw_qkv", "dw_bias"):
        if got[n] is not None:
            assert torch.equal(got[n], again[n]), f"{n}: two calls differ (fixed-order sums expected)"
    assert torch.equal(got["dx"], again["dx"])
    sub = inp
    dx_gpu = got["dx"]
    if ia is not None:
        keep = torch.zeros(inp["x"].shape[:2], dtype=torch.bool)
        keep[ia[:, None], ib[None, :]] = True
        assert bool((dx_gpu.cpu()[~keep] == 0).all()), "dx must vanish where the upstream gradient is zero"
        dx_gpu = dx_gpu[ia][:, ib]
        sub = dict(inp)
        sub["x"] = inp["x"][ia][:, ib]
        for n in ("dq", "dk", "dv"):
            if inp[n] is not None:
                sub[n] = inp[n][ia][:, ib]
        if inp["dbias"] is not None:
            sub["dbias"] = (inp["dbias"][:, ib][:, :, ia] if bias_transpose else inp["dbias"][:, ia][:, :, ib])
    x, gamma, beta = f64(sub["x"]), f64(sub["gamma"]), f64(sub["beta"])
    wq, wb = f64(sub["w_qkv"]), f64(sub["w_bias"])
    ref = oracle.ln_proj_bwd(x, gamma, beta, sub["eps"], wq, wb, H, D, bias_transpose,
                             f64(sub["dq"]), f64(sub["dk"]), f64(sub["dv"]), f64(sub["dbias"]))
    A, B, C = x.shape
    errs = {}
    g, r = f64(dx_gpu).reshape(A * B, C), ref["dx"].reshape(A * B, C)
    assert np.all(np.isfinite(g))
    if mode == "bf16":
        G = upstream_by_token(sub, bias_transpose)
        W = np.concatenate([w for w in (wq, wb) if w is not None], axis=0)
        n_qkv = 0 if wq is None else wq.shape[0]
        Eb = np.zeros((A * B, C))
        if wb is not None:
            Eb = 2.0 ** -8 * (np.abs(G[:, n_qkv:]) @ np.abs(wb))
        E = (Eb + W.shape[0] * 2.0 ** -24 * (np.abs(G) @ np.abs(W))).max(axis=1, keepdims=True)
        _, xhat, _, rstd = oracle.layer_norm(x, gamma, beta, sub["eps"])
        xh = xhat.reshape(A * B, C)
        tol = 2.0 ** -7 * np.abs(r) + 1.2 * rstd.reshape(-1, 1) * np.abs(gamma).max() * E * (2 + np.abs(xh)) + 1e-6
    else:
        tol = FP32_REL * np.abs(r).max(axis=1, keepdims=True) + 1e-7
    err = np.abs(g - r)
    errs["dx"] = float((err / tol).max())
    assert np.all(err <= tol), f"dx: worst err/tol {errs['dx']:.3f}"
    rel = BF16_RED_REL if mode == "bf16" else FP32_REL
    for n in ("dgamma", "dbeta", "dw_qkv", "dw_bias"):
        if ref[n] is None:
            assert got[n] is None
            continue
        e = np.abs(f64(got[n]) - ref[n]).max() / np.abs(ref[n]).max()
        errs[n] = float(e)
        assert e <= rel, f"{n}: max err / max|ref| = {e:.2e} > {rel}"
    print("bwd", errs, flush=True)
    return errs


def test_bwd_fp32_workload():
    w = PROJ_WORKLOADS["pair_proj_fp32_n64"]
    banner("bwd " + w.name)
    check_bwd(generate_proj_workload(w), 0, "fp32")


@pytest.mark.parametrize("bt", [0, 1])
@pytest.mark.parametrize("N", [50, 97])
def test_bwd_bf16_pair_c128(N, bt):
    banner(f"bwd bf16 pair N={N} C=128 bt={bt}")
    check_bwd(generate_proj(N, N, 128, 4, 32, dtype=torch.bfloat16, seed=N + 7 * bt), bt, "bf16")


@pytest.mark.parametrize("A,B,C,H,D,qkv,bias,bt", [
    (37, 45, 64, 8, 8, True, False, 0),
    (33, 33, 64, 4, 32, False, True, 1),
    (40, 40, 32, 1, 8, True, True, 0),
    (40, 40, 32, 1, 8, True, True, 1),
    (29, 29, 128, 2, 64, True, True, 1),
    (1, 1, 128, 4, 32, True, True, 0),
])
def test_bwd_bf16_shapes(A, B, C, H, D, qkv, bias, bt):
    banner(f"bwd bf16 A={A} B={B} C={C} H={H} D={D} qkv={qkv} bias={bias} bt={bt}")
    check_bwd(generate_proj(A, B, C, H, D, dtype=torch.bfloat16, qkv=qkv, bias=bias, seed=A + C), bt, "bf16")


@pytest.mark.parametrize("A,B,C,H,D,bt", [(37, 37, 64, 8, 8, 0), (29, 29, 128, 2, 64, 1)])
def test_bwd_ignores_workspace_contents(A, B, C, H, D, bt):
    """The workspace (fixed-order partial sums) may hold anything on entry: a
    workspace of NaN bytes gives the same bits as a zeroed one."""
    import af3_attention_amd as ea
    banner(f"bwd workspace contents A={A} B={B} C={C} H={H} D={D} bt={bt}")
    inp = generate_proj(A, B, C, H, D, dtype=torch.bfloat16, qkv=True, bias=True, seed=A * 3 + C)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    fw = ea.ln_proj_fwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], heads=H, head_dim=D,
                        bias_transpose=bt, eps=inp["eps"])
    nbytes = ea.ln_proj_bwd_workspace_bytes(A, B, C, H, D)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        outs.append(ea.ln_proj_bwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], fw["mean"], fw["rstd"],
                                   g["dq"], g["dk"], g["dv"], g["dbias"], heads=H, head_dim=D, bias_transpose=bt,
                                   workspace=ws))
    torch.cuda.synchronize()
    for n in outs[0]:
        if outs[0][n] is None:
            continue
        assert bool(torch.isfinite(outs[1][n]).all()), f"{n}: non-finite with a NaN-filled workspace"
        assert torch.equal(outs[0][n], outs[1][n]), f"{n}: depends on the workspace contents"


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
@pytest.mark.parametrize("A,C,H,D,bt", [(20, 96, 2, 16, 1), (9, 256, 4, 32, 0)])
def test_bwd_vector_kernel_shapes(A, C, H, D, bt, mode):
    banner(f"bwd {mode} vector A={A} C={C} H={H} D={D} bt={bt}")
    check_bwd(generate_proj(A, A, C, H, D, dtype=dtype_of(mode), seed=C + 2 * A), bt, mode)


@pytest.mark.parametrize("name", ["pair_proj_bf16_n384", "pair_proj_end_bf16_n768", "msa_proj_bf16_s512_n384"])
def test_bwd_bf16_workloads_sampled(name):
    """Full sizes in the benchmark's launch configuration, upstream gradients zero
    outside a 64 x 64 token sub-grid: the reductions then equal the sub-grid's
    exactly, dx matches on the sub-grid and vanishes elsewhere."""
    w = PROJ_WORKLOADS[name]
    banner("bwd " + w.name)
    inp = generate_proj_workload(w)
    ia, ib = sample_axis(w.a, 64, 3), sample_axis(w.b, 64, 4)
    keep = torch.zeros((w.a, w.b), dtype=torch.bool)
    keep[ia[:, None], ib[None, :]] = True
    for n in ("dq", "dk", "dv"):
        if inp[n] is not None:
            inp[n] = inp[n] * keep[:, :, None, None].to(inp[n].dtype)
    if inp["dbias"] is not None:
        kb = keep.T if w.bias_transpose else keep
        inp["dbias"] = inp["dbias"] * kb[None].float()
    check_bwd(inp, w.bias_transpose, "bf16", ia, ib)


def test_autograd_matches_entry_points():
    """LNProjFunction's gradients equal the C entry points' (same kernels, casts of dW)."""
    import af3_attention_amd as ea
    banner("autograd")
    inp = bwd_inputs_gpu(generate_proj(24, 24, 128, 4, 32, dtype=torch.bfloat16, seed=42))
    x = inp["x"].clone().requires_grad_(True)
    gamma = inp["gamma"].clone().requires_grad_(True)
    beta = inp["beta"].clone().requires_grad_(True)
    wq = inp["w_qkv"].clone().requires_grad_(True)
    wb = inp["w_bias"].clone().requires_grad_(True)
    q, k, v, b = ea.ln_proj(x, gamma, beta, wq, wb, heads=4, head_dim=32)
    loss = ((q.float() * inp["dq"].float()).sum() + (k.float() * inp["dk"].float()).sum()
            + (v.float() * inp["dv"].float()).sum() + (b.float() * inp["dbias"]).sum())
    loss.backward()
    fw = ea.ln_proj_fwd(inp["x"], inp["gamma"], inp["beta"], inp["w_qkv"], inp["w_bias"], heads=4, head_dim=32)
    ref = ea.ln_proj_bwd(inp["x"], inp["gamma"], inp["beta"], inp["w_qkv"], inp["w_bias"], fw["mean"], fw["rstd"],
                         inp["dq"], inp["dk"], inp["dv"], inp["dbias"], heads=4, head_dim=32)
    torch.cuda.synchronize()
    assert torch.equal(x.grad, ref["dx"])
    assert torch.equal(gamma.grad, ref["dgamma"]) and torch.equal(beta.grad, ref["dbeta"])
    assert torch.equal(wq.grad, ref["dw_qkv"].to(torch.bfloat16))
    assert torch.equal(wb.grad, ref["dw_bias"].to(torch.bfloat16))


@pytest.mark.parametrize("bt", [0, 1])
def test_pair_to_attention_chain(bt):
    """The pair tensor's path end to end: layer norm + projections, then triangle
    attention (starting node, or ending node with bt = 1), fwd and bwd on the GPU,
    against the oracle chain; gradients to 5e-2 of their max norm."""
    import af3_attention_amd as ea
    banner(f"chain bt={bt}")
    N, C, H, D = 40, 128, 4, 32
    inp = generate_proj(N, N, C, H, D, dtype=torch.bfloat16, seed=100 + bt)
    g = bwd_inputs_gpu(inp)
    fw = ea.ln_proj_fwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], heads=H, head_dim=D,
                        bias_transpose=bt)
    o, lse = ea.evoattn_fwd(fw["q"], fw["k"], fw["v"], fw["bias"], None, transpose=bt)
    dout = g["dq"]  # any seeded [N, N, H, d] tensor serves as the gradient of o
    dq, dk, dv, db = ea.evoattn_bwd(fw["q"], fw["k"], fw["v"], fw["bias"], None, o, lse, dout, transpose=bt)
    gb = ea.ln_proj_bwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], fw["mean"], fw["rstd"], dq, dk, dv,
                        db, heads=H, head_dim=D, bias_transpose=bt)
    torch.cuda.synchronize()
    x, gm, bt_, wq, wb = (f64(inp[n]) for n in ("x", "gamma", "beta", "w_qkv", "w_bias"))
    rf = oracle.ln_proj_fwd(x, gm, bt_, inp["eps"], wq, wb, H, D, bt)
    ro, _ = oracle.fwd(rf["q"], rf["k"], rf["v"], rf["bias"], None, bt)
    rdq, rdk, rdv, rdb = oracle.bwd(rf["q"], rf["k"], rf["v"], rf["bias"], None, f64(inp["dq"]), bt)
    rg = oracle.ln_proj_bwd(x, gm, bt_, inp["eps"], wq, wb, H, D, bt, rdq, rdk, rdv, rdb)
    assert np.abs(f64(o) - ro).max() <= 2e-2 * max(1.0, np.abs(ro).max())
    for n in ("dx", "dgamma", "dbeta", "dw_qkv", "dw_bias"):
        e = np.abs(f64(gb[n]) - rg[n]).max() / np.abs(rg[n]).max()
        print(n, f"{e:.2e}", flush=True)
        assert e <= 5e-2, n
