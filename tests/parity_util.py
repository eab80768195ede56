"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on the
same seeded inputs and compare them to the stated tolerances.

Tolerances (from the statement of the target for this operator):
  fp32 mode: every output within 1e-4 max abs of the fp64 oracle.
  bf16 mode: O within 2e-2 max abs; each gradient within 5e-2 of the oracle,
             measured as max|g - g_ref| / max|g_ref| ("relative to max norm");
             lse within 1e-3 max abs (a tolerance the statement leaves open; the
             kernels sum the fp32 probabilities, so lse carries only fp32
             rounding of the logits and the sum).
"""
import numpy as np
import torch

import oracle

FP32_ATOL = 1e-4
BF16_O_ATOL = 2e-2
BF16_GRAD_REL = 5e-2
BF16_LSE_ATOL = 1e-3


def to_np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def gpu_fwd_bwd(inp, dout=None, need_dbias=True):
    import af3_attention_amd as ea
    dev = torch.device("cuda:0")
    g = {x: (None if inp[x] is None else inp[x].to(dev)) for x in ("q", "k", "v", "bias", "mask", "dout")}
    if dout is not None:
        g["dout"] = dout.to(dev)
    t = bool(inp["transpose"])
    o, lse = ea.evoattn_fwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], t)
    dq, dk, dv, db = ea.evoattn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, lse, g["dout"], t,
                                    need_dbias=need_dbias)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dbias": db}


def oracle_fwd_bwd(inp, rows=None, dout=None):
    q, k, v, b, m = (to_np(inp[x]) for x in ("q", "k", "v", "bias", "mask"))
    do = to_np(inp["dout"] if dout is None else dout)
    t = inp["transpose"]
    o, lse = oracle.fwd(q, k, v, b, m, t, rows=rows)
    dq, dk, dv, db = oracle.bwd(q, k, v, b, m, do, t, rows=rows)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dbias": db}


def row_select(x, rows, transpose, kind):
    """Pick attention rows from an output: [R,N,H,d] (or [N,R,H,d] transposed) or lse [R,H,N]."""
    if kind == "lse":
        return x[rows]
    return x[:, rows] if transpose else x[rows]


def compare(gpu, ref, mode, transpose=0, rows=None, check_dbias=True):
    """Returns a dict of errors; raises AssertionError with all errors if any exceeds tolerance."""
    errs, bad = {}, []
    for name in ("o", "lse", "dq", "dk", "dv", "dbias"):
        if name == "dbias" and not check_dbias:
            continue
        g = to_np(gpu[name])
        r = ref[name]
        if rows is not None and name != "dbias":
            g = row_select(g, rows, transpose, "lse" if name == "lse" else "t")
            r = row_select(r, rows, transpose, "lse" if name == "lse" else "t")
        # -inf must match exactly (fully masked rows)
        if name == "lse":
            ninf = np.isneginf(r)
            if not np.array_equal(ninf, np.isneginf(g)):
                bad.append(f"lse -inf pattern differs")
            g = np.where(ninf, 0.0, g)
            r = np.where(ninf, 0.0, r)
        if not np.all(np.isfinite(g)):
            bad.append(f"{name}: non-finite values")
            continue
        diff = float(np.max(np.abs(g - r))) if g.size else 0.0
        if mode == "fp32":
            err, tol = diff, FP32_ATOL
        elif name == "o":
            err, tol = diff, BF16_O_ATOL
        elif name == "lse":
            err, tol = diff, BF16_LSE_ATOL
        else:
            scale = float(np.max(np.abs(r))) if r.size else 0.0
            err, tol = (diff / scale if scale > 0 else diff), BF16_GRAD_REL
        errs[name] = err
        if not err <= tol:
            bad.append(f"{name}: err {err:.3e} > tol {tol:.1e}")
    assert not bad, f"{bad}; all errors: {errs}"
    return errs


def sample_rows(R, count, seed=0):
    """First, last and `count` random rows, sorted."""
    g = torch.Generator().manual_seed(seed + 1234)
    pick = set(torch.randperm(R, generator=g)[:count].tolist()) | {0, R - 1}
    return sorted(pick)


def masked_dout(dout, rows, transpose):
    """dO with every attention row outside `rows` set to zero, so those rows add nothing to dBias."""
    d = torch.zeros_like(dout)
    if transpose:
        d[:, rows] = dout[:, rows]
    else:
        d[rows] = dout[rows]
    return d
