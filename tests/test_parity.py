"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the
same seeded inputs.  Small sizes compare every element; full workload sizes
compare sampled rows (forward rows are independent, and with dO zero outside
the sample the GPU's dBias must equal the sample's exact sum)."""
import math

import numpy as np
import pytest
import torch

from parity_util import (compare, gpu_fwd_bwd, masked_dout, oracle_fwd_bwd, sample_rows)
from workloads import WORKLOADS, generate, generate_workload

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[parity] {msg}", flush=True)


# ---------------------------------------------------------------- small, every element

def test_fp32_workload_full():
    """The small fp32 workload: N=64, 64 rows, H=4, d=32, no mask; every output to 1e-4."""
    w = WORKLOADS["tri_start_fp32_n64"]
    banner(w.name)
    inp = generate_workload(w)
    errs = compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "fp32")
    print(errs)


@pytest.mark.parametrize("transpose", [0, 1])
@pytest.mark.parametrize("R,N,H,D", [(9, 100, 4, 32), (33, 70, 2, 32), (5, 130, 3, 16), (7, 65, 2, 64)])
def test_fp32_ragged(R, N, H, D, transpose):
    banner(f"fp32 R={R} N={N} H={H} D={D} t={transpose}")
    inp = generate(R, N, H, D, dtype=torch.float32, transpose=transpose, bias_std=math.sqrt(2),
                   mask_kind="tail_fixed", mask_frac=0.15, seed=R + N)
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "fp32", transpose)


@pytest.mark.parametrize("transpose", [0, 1])
@pytest.mark.parametrize("R,N,H,D", [(50, 100, 4, 32), (17, 200, 4, 32), (64, 64, 4, 32), (3, 257, 2, 32)])
def test_bf16_ragged_triangle(R, N, H, D, transpose):
    banner(f"bf16 R={R} N={N} H={H} D={D} t={transpose}")
    inp = generate(R, N, H, D, dtype=torch.bfloat16, transpose=transpose, bias_std=math.sqrt(2),
                   mask_kind="tail_uniform", mask_frac=0.15, seed=R * 7 + N)
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "bf16", transpose)


@pytest.mark.parametrize("R,N,H,D,transpose", [(150, 100, 2, 32, 0), (150, 100, 2, 32, 1), (200, 20, 3, 16, 0),
                                                 (200, 20, 3, 16, 1), (130, 257, 4, 32, 0), (300, 72, 4, 8, 0)])
def test_bf16_rows_per_workgroup(R, N, H, D, transpose):
    """More (row, head) pairs than compute units, so the persistent fused backward's
    workgroups walk several rows (row changes with a ragged last key tile, one key
    tile only, and d = 8 and 16)."""
    banner(f"bf16 rows per workgroup R={R} N={N} H={H} D={D} t={transpose}")
    inp = generate(R, N, H, D, dtype=torch.bfloat16, transpose=transpose, bias_std=math.sqrt(2),
                   mask_kind="tail_uniform", mask_frac=0.15, seed=R * 3 + N + D)
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "bf16", transpose)


@pytest.mark.parametrize("transpose", [0, 1])
def test_bwd_ignores_workspace_contents(transpose):
    """The backward's workspace (tiled bias copies, per-row operands, dBias partial
    sums) may hold anything on entry: a workspace of NaN bytes gives the same bits
    as a zeroed one."""
    import af3_attention_amd as ea
    R, N, H, D = 17, 200, 4, 32
    banner(f"bwd workspace contents R={R} N={N} t={transpose}")
    inp = generate(R, N, H, D, dtype=torch.bfloat16, transpose=transpose, bias_std=math.sqrt(2),
                   mask_kind="tail_uniform", mask_frac=0.15, seed=5)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, lse = ea.evoattn_fwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], bool(transpose))
    nbytes = ea.evoattn_bwd_workspace_bytes(R, N, H, D)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        outs.append(ea.evoattn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, lse, g["dout"],
                                   bool(transpose), workspace=ws))
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dbias"), *outs):
        assert bool(torch.isfinite(b).all()), f"{name}: non-finite with a NaN-filled workspace"
        assert torch.equal(a, b), f"{name}: depends on the workspace contents"


@pytest.mark.parametrize("R,N,H,D", [(40, 72, 8, 8), (21, 150, 8, 8), (12, 96, 4, 16), (10, 80, 2, 64)])
def test_bf16_msa_like_and_other_dims(R, N, H, D):
    banner(f"bf16 msa-like R={R} N={N} H={H} D={D}")
    inp = generate(R, N, H, D, dtype=torch.bfloat16, bias_std=1.0, mask_kind="random_positions",
                   mask_frac=0.2, seed=R + 3 * N)
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "bf16")


@pytest.mark.parametrize("R,N,H,D", [(24, 96, 1, 32), (6, 64, 16, 16), (5, 400, 16, 32)])
def test_bf16_one_and_sixteen_heads(R, N, H, D):
    banner(f"bf16 heads R={R} N={N} H={H} D={D}")
    inp = generate(R, N, H, D, dtype=torch.bfloat16, bias_std=math.sqrt(2), mask_kind="tail_uniform",
                   mask_frac=0.15, seed=R + N + H)
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "bf16")


@pytest.mark.parametrize("R,N,transpose", [(40, 200, 0), (12, 520, 1)])
def test_bwd_without_dbias_matches(R, N, transpose):
    """Skipping dBias (as autograd does for a bias that needs no gradient) leaves dQ, dK,
    dV bit for bit as they are with it, on the fused (N <= 384) and the separate paths."""
    import af3_attention_amd as ea
    banner(f"bwd without dBias R={R} N={N} t={transpose}")
    inp = generate(R, N, 4, 32, dtype=torch.bfloat16, transpose=transpose, bias_std=math.sqrt(2),
                   mask_kind="tail_uniform", mask_frac=0.15, seed=R + N)
    g = {x: inp[x].cuda() for x in ("q", "k", "v", "bias", "mask", "dout")}
    t = bool(transpose)
    o, lse = ea.evoattn_fwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], t)
    with_db = ea.evoattn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, lse, g["dout"], t, need_dbias=True)
    without = ea.evoattn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, lse, g["dout"], t, need_dbias=False)
    torch.cuda.synchronize()
    assert without[3] is None
    for a, b in zip(with_db[:3], without[:3]):
        assert torch.equal(a, b)


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("dtype,mode", [(torch.float32, "fp32"), (torch.bfloat16, "bf16")])
def test_single_position(dtype, mode):
    banner(f"N=1 {mode}")
    inp = generate(6, 1, 2, 32, dtype=dtype, mask_kind="none", seed=4)
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), mode)


@pytest.mark.parametrize("dtype,mode", [(torch.float32, "fp32"), (torch.bfloat16, "bf16")])
def test_single_row_and_no_bias_no_mask(dtype, mode):
    banner(f"R=1, no bias, no mask {mode}")
    inp = generate(1, 90, 4, 32, dtype=dtype, mask_kind="none", seed=5, with_bias=False)
    got = gpu_fwd_bwd(inp, need_dbias=True)
    compare(got, oracle_fwd_bwd(inp), mode)


@pytest.mark.parametrize("dtype,mode", [(torch.float32, "fp32"), (torch.bfloat16, "bf16")])
def test_fully_masked_rows(dtype, mode):
    """Rows whose keys are all masked give O = 0, lse = -inf and add nothing to any gradient."""
    banner(f"fully masked rows {mode}")
    inp = generate(6, 80, 2, 32, dtype=dtype, mask_kind="tail_fixed", mask_frac=0.1, seed=6)
    inp["mask"][2, :] = float("-inf")
    inp["mask"][5, :] = float("-inf")
    got = gpu_fwd_bwd(inp)
    ref = oracle_fwd_bwd(inp)
    compare(got, ref, mode)
    o = got["o"].float().cpu()
    assert torch.all(o[2] == 0) and torch.all(o[5] == 0)
    assert torch.all(torch.isneginf(got["lse"][2].cpu()))
    for g in ("dq", "dk", "dv"):
        assert torch.all(got[g][2].float().cpu() == 0), g


def test_finite_mask_values():
    """Finite (non -inf) additive mask entries are added to the logits like any bias."""
    banner("finite mask values")
    inp = generate(8, 96, 2, 32, dtype=torch.float32, mask_kind="none", seed=8)
    inp["mask"] = torch.randn(8, 96, generator=torch.Generator().manual_seed(1)) * 2.0
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "fp32")


def test_large_logits_stay_finite():
    """Logits of magnitude ~100 (large bias) must not overflow the online softmax."""
    banner("large logits")
    inp = generate(4, 128, 2, 32, dtype=torch.float32, bias_std=60.0, mask_kind="tail_fixed",
                   mask_frac=0.1, seed=9)
    compare(gpu_fwd_bwd(inp), oracle_fwd_bwd(inp), "fp32")


def test_bf16_softmax_reference_paths():
    """bf16 path: rows whose first key block is masked, rows whose later logits
    exceed the first block's by ~90 (the exact recompute path), fully masked rows."""
    banner("bf16 softmax reference paths")
    inp = generate(6, 200, 2, 32, dtype=torch.bfloat16, mask_kind="none", seed=12)
    bias = inp["bias"].float()
    bias[0, :, :32] = -90.0  # head 0: every query's first 32 keys far below the rest
    inp["bias"] = bias.to(torch.bfloat16)
    mask = torch.zeros(6, 200)
    mask[1, :40] = float("-inf")  # first block dead, second partly
    mask[2, :] = float("-inf")    # fully masked
    mask[4, 150:] = float("-inf")
    inp["mask"] = mask
    got = gpu_fwd_bwd(inp)
    compare(got, oracle_fwd_bwd(inp), "bf16")
    assert torch.all(got["o"][2].float().cpu() == 0)
    assert torch.all(torch.isneginf(got["lse"][2].cpu()))


# ---------------------------------------------------------------- full sizes, sampled rows

FULL = [
    ("tri_start_bf16_n384", 0, 24),
    ("tri_end_bf16_n768", None, 8),
    ("msa_row_bf16_s512_n384", None, 24),
    ("tri_long_bf16_n1536", 0, 3),
    ("tri_long_bf16_n1536", 1, 3),
]


@pytest.mark.parametrize("name,transpose,count", FULL)
def test_full_size_sampled_rows(name, transpose, count):
    w = WORKLOADS[name]
    t = w.transpose if transpose is None else transpose
    banner(f"{name} transpose={t} sampled rows={count}")
    inp = generate_workload(w, transpose=t)
    rows = sample_rows(w.rows, count)
    dout = masked_dout(inp["dout"], rows, t)
    got = gpu_fwd_bwd(inp, dout=dout)
    ref = oracle_fwd_bwd(inp, rows=rows, dout=dout)
    errs = compare(got, ref, "bf16", t, rows=rows)
    print(errs, flush=True)


@pytest.mark.parametrize("transpose", [0, 1])
def test_n2048_sampled_rows(transpose):
    """N = R = 2048 (the size at which the materialised reference of the memory curve runs
    out of memory on one MI355X): sampled rows against the oracle."""
    banner(f"N=2048 transpose={transpose} sampled rows=4")
    inp = generate(2048, 2048, 4, 32, dtype=torch.bfloat16, transpose=transpose, bias_std=math.sqrt(2.0),
                   mask_kind="tail_fixed", mask_frac=0.05, seed=transpose)
    rows = sample_rows(2048, 4)
    dout = masked_dout(inp["dout"], rows, transpose)
    got = gpu_fwd_bwd(inp, dout=dout)
    ref = oracle_fwd_bwd(inp, rows=rows, dout=dout)
    errs = compare(got, ref, "bf16", transpose, rows=rows)
    print(errs, flush=True)


def test_dbias_bitwise_deterministic():
    """dBias is bit-identical over repeated backward calls, with other work in between."""
    import af3_attention_amd as ea
    w = WORKLOADS["tri_start_bf16_n384"]
    banner("dbias determinism x20")
    inp = generate_workload(w, device="cuda:0")
    o, lse = ea.evoattn_fwd(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], False)
    first = None
    for i in range(20):
        _, _, _, db = ea.evoattn_bwd(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], o, lse,
                                     inp["dout"], False)
        if i % 5 == 4:  # unrelated work on the same stream
            torch.randn(1 << 22, device="cuda:0").sum()
        if first is None:
            first = db.clone()
        else:
            assert torch.equal(db.view(torch.int32), first.view(torch.int32)), f"run {i} differs"
