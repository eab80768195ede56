"""Seeded synthetic inputs for the 3D (triangle / MSA-row) attention workloads.

This module only draws random numbers and lays them out. It holds none of the
attention arithmetic, so both the CPU oracle tests and the HIP path use it
without sharing any compute code.

Workloads stand in for the MegaFold pages' training regimes (gist.science
"MegaFold" technical summary, Problemstellung and Ergebnisse): AF3 training
crops of a few hundred residues, lengths past the ~590-residue point where the
materialised baseline runs out of memory, and the ~1450-residue maximum reached
with the memory-efficient kernel.  No dataset items are used.

Conventions (kernel frame):
  q, k, v, dO : element (r, p, h, c) = row r, position p, head h, channel c.
                Physical layout [R, N, H, d] when transpose == 0 and
                [N, R, H, d] when transpose == 1 (ending-node attention runs
                along the first axis of the pair tensor).
  bias        : [H, N, N], bias[h, j, k] for query j and key k, shared by all rows.
  mask        : [R, N] additive fp32 (0 or -inf), mask[r, k] for key k of row r.

Draw order with one torch CPU generator seeded with `seed`: q, k, v, bias, dO,
then the mask draws.  Values are drawn in fp32 and cast to the compute dtype
with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int          # R: attention rows (pair rows, or MSA rows)
    n: int             # N: positions per row (queries = keys)
    heads: int         # H
    head_dim: int      # d
    dtype: str         # "fp32" or "bf16"
    transpose: int     # 0 = starting node / MSA row, 1 = ending node
    bias_std: float    # standard deviation of bias entries
    mask_kind: str     # "none", "tail_uniform", "tail_fixed", "random_positions"
    mask_frac: float   # parameter of the mask recipe
    desc: str = ""
    variants: tuple = field(default=(0,))  # transpose flags run back to back

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def flops_fwd(self) -> float:
        """4 * R * N^2 * H * d: two N x N x d contractions (Q K^T, P V) per row and head."""
        return 4.0 * self.rows * self.n * self.n * self.heads * self.head_dim

    def flops_fwd_bwd(self) -> float:
        """Forward 4 R N^2 H d plus backward 10 R N^2 H d (Q K^T recompute, dO V^T,
        P^T dO, dS^T Q, dS K): five N x N x d contractions."""
        return 14.0 * self.rows * self.n * self.n * self.heads * self.head_dim


WORKLOADS = {
    # Small fp32 case the oracle finishes in seconds.
    "tri_start_fp32_n64": Workload(
        "tri_start_fp32_n64", 64, 64, 4, 32, "fp32", 0, 1.0, "none", 0.0,
        "starting-node triangle attention, fp32, N=64 H=4 d=32, no mask"),
    # AF3 training crop: the headline configuration.
    "tri_start_bf16_n384": Workload(
        "tri_start_bf16_n384", 384, 384, 4, 32, "bf16", 0, math.sqrt(2.0), "tail_uniform", 0.15,
        "starting-node triangle attention, bf16, N=384 H=4 d=32, tail key mask of 0-15%"),
    # Ending node on the transposed pair layout.
    "tri_end_bf16_n768": Workload(
        "tri_end_bf16_n768", 768, 768, 4, 32, "bf16", 1, math.sqrt(2.0), "tail_fixed", 0.10,
        "ending-node triangle attention, bf16, N=768 H=4 d=32, 10% tail key mask"),
    # MSA row attention with pair bias.
    "msa_row_bf16_s512_n384": Workload(
        "msa_row_bf16_s512_n384", 512, 384, 8, 8, "bf16", 0, 1.0, "random_positions", 0.20,
        "MSA row attention with pair bias, bf16, S=512 N=384 H=8 d=8, 20% random positions masked"),
    # Long sequence: starting and ending node back to back.
    "tri_long_bf16_n1536": Workload(
        "tri_long_bf16_n1536", 1536, 1536, 4, 32, "bf16", 0, math.sqrt(2.0), "tail_fixed", 0.05,
        "long-sequence triangle attention, bf16, N=1536 H=4 d=32, 5% tail key mask, "
        "starting then ending node", variants=(0, 1)),
}


def physical_shape(rows: int, n: int, heads: int, head_dim: int, transpose: int):
    return (n, rows, heads, head_dim) if transpose else (rows, n, heads, head_dim)


def make_mask(kind: str, frac: float, rows: int, n: int, gen: torch.Generator):
    """Additive key mask [R, N] fp32 (0 or -inf), or None.

    tail_uniform     : m = floor(frac * u * N), u ~ U[0,1); last m keys masked in every row.
    tail_fixed       : m = floor(frac * N); last m keys masked in every row.
    random_positions : each row independently masks floor(frac * N) positions chosen by randperm.
    """
    if kind == "none":
        return None
    mask = torch.zeros(rows, n, dtype=torch.float32)
    if kind == "tail_uniform":
        u = torch.rand(1, generator=gen).item()
        m = int(math.floor(frac * u * n))
    elif kind == "tail_fixed":
        m = int(math.floor(frac * n))
    elif kind == "random_positions":
        m = int(math.floor(frac * n))
        for r in range(rows):
            idx = torch.randperm(n, generator=gen)[:m]
            mask[r, idx] = float("-inf")
        return mask
    else:
        raise ValueError(f"unknown mask kind {kind!r}")
    if m > 0:
        mask[:, n - m:] = float("-inf")
    return mask


def generate(rows: int, n: int, heads: int, head_dim: int, *, dtype=torch.bfloat16,
             transpose: int = 0, bias_std: float = 1.0, mask_kind: str = "none",
             mask_frac: float = 0.0, seed: int = 0, device="cpu", with_bias: bool = True):
    """Draw one seeded input set.  Returns a dict with q, k, v, bias, mask, dout.

    Tensors are drawn on the CPU (so the values do not depend on the device)
    and then moved to `device`.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    shape = physical_shape(rows, n, heads, head_dim, transpose)
    q = torch.randn(shape, generator=gen, dtype=torch.float32)
    k = torch.randn(shape, generator=gen, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, dtype=torch.float32)
    bias = None
    if with_bias:
        bias = torch.randn((heads, n, n), generator=gen, dtype=torch.float32) * bias_std
    dout = torch.randn(shape, generator=gen, dtype=torch.float32)
    mask = make_mask(mask_kind, mask_frac, rows, n, gen)

    def cast(t):
        if t is None:
            return None
        return t.to(dtype).to(device).contiguous()

    return {
        "q": cast(q), "k": cast(k), "v": cast(v), "bias": cast(bias), "dout": cast(dout),
        "mask": None if mask is None else mask.to(device).contiguous(),
        "rows": rows, "n": n, "heads": heads, "head_dim": head_dim, "transpose": transpose,
    }


def generate_workload(w: Workload, *, transpose: int | None = None, seed: int = 0, device="cpu"):
    t = w.transpose if transpose is None else transpose
    return generate(w.rows, w.n, w.heads, w.head_dim, dtype=w.torch_dtype, transpose=t,
                    bias_std=w.bias_std, mask_kind=w.mask_kind, mask_frac=w.mask_frac,
                    seed=seed, device=device)


# ---------------------------------------------------------------- LayerNorm + projections

@dataclass(frozen=True)
class ProjWorkload:
    """The fused layer norm + projection step that produces the attention inputs.

    x is [A, B, c] (pair tensor: A = B = N, c = pair channels; MSA: A = S rows,
    B = N, c = MSA channels).  With qkv, the projection writes q, k, v of
    [A, B, H, d]; with bias (pair tensor only) it writes the pair bias [H, N, N]."""
    name: str
    a: int
    b: int
    channels: int
    heads: int
    head_dim: int
    dtype: str
    qkv: bool
    bias: bool
    bias_transpose: int = 0
    desc: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def tokens(self) -> int:
        return self.a * self.b

    @property
    def outputs(self) -> int:
        return (3 * self.heads * self.head_dim if self.qkv else 0) + (self.heads if self.bias else 0)


PROJ_WORKLOADS = {
    "pair_proj_fp32_n64": ProjWorkload(
        "pair_proj_fp32_n64", 64, 64, 128, 4, 32, "fp32", True, True, 0,
        "pair tensor N=64, c=128 -> q, k, v (H=4, d=32) and pair bias, fp32"),
    # The step that feeds the headline attention workload (starting node, N=384).
    "pair_proj_bf16_n384": ProjWorkload(
        "pair_proj_bf16_n384", 384, 384, 128, 4, 32, "bf16", True, True, 0,
        "pair tensor N=384, c=128 -> q, k, v (H=4, d=32) and pair bias, bf16"),
    "pair_proj_end_bf16_n768": ProjWorkload(
        "pair_proj_end_bf16_n768", 768, 768, 128, 4, 32, "bf16", True, True, 1,
        "pair tensor N=768, c=128 -> q, k, v and the transposed pair bias (ending node), bf16"),
    "msa_proj_bf16_s512_n384": ProjWorkload(
        "msa_proj_bf16_s512_n384", 512, 384, 64, 8, 8, "bf16", True, False, 0,
        "MSA tensor S=512 N=384, c=64 -> q, k, v (H=8, d=8), bf16"),
}


def generate_proj(a: int, b: int, channels: int, heads: int, head_dim: int, *, dtype=torch.bfloat16,
                  qkv: bool = True, bias: bool = True, seed: int = 0, device="cpu"):
    """Draw one seeded input set for layer norm + projections.

    Draw order with one torch CPU generator: x, per-token scale, per-token
    offset, gamma, beta, w_qkv, w_bias, dq, dk, dv, dbias.  Tokens get their own
    offset (N(0,1)) and scale (exp of N(0, 0.5^2)) so the normalisation has
    real work to do; gamma ~ 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2) (fp32);
    weights ~ N(0, 1/c) (fan-in scaling), cast to the compute dtype; upstream
    gradients ~ N(0, 1) (dbias fp32, as the attention backward produces it)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    hd = heads * head_dim
    x = torch.randn((a, b, channels), generator=gen, dtype=torch.float32)
    scale = torch.exp(0.5 * torch.randn((a, b, 1), generator=gen, dtype=torch.float32))
    offset = torch.randn((a, b, 1), generator=gen, dtype=torch.float32)
    x = x * scale + offset
    gamma = 1.0 + 0.1 * torch.randn(channels, generator=gen, dtype=torch.float32)
    beta = 0.1 * torch.randn(channels, generator=gen, dtype=torch.float32)
    w_qkv = torch.randn((3 * hd, channels), generator=gen, dtype=torch.float32) / math.sqrt(channels)
    w_bias = torch.randn((heads, channels), generator=gen, dtype=torch.float32) / math.sqrt(channels)
    grads = [torch.randn((a, b, heads, head_dim), generator=gen, dtype=torch.float32) for _ in range(3)]
    dbias = torch.randn((heads, a, b), generator=gen, dtype=torch.float32)

    def cast(t, dt=dtype):
        return t.to(dt).to(device).contiguous()

    return {
        "x": cast(x), "gamma": cast(gamma, torch.float32), "beta": cast(beta, torch.float32),
        "w_qkv": cast(w_qkv) if qkv else None, "w_bias": cast(w_bias) if bias else None,
        "dq": cast(grads[0]) if qkv else None, "dk": cast(grads[1]) if qkv else None,
        "dv": cast(grads[2]) if qkv else None,
        "dbias": cast(dbias, torch.float32) if bias else None,
        "eps": 1e-5, "heads": heads, "head_dim": head_dim,
    }


def generate_proj_workload(w: ProjWorkload, *, seed: int = 0, device="cpu"):
    out = generate_proj(w.a, w.b, w.channels, w.heads, w.head_dim, dtype=w.torch_dtype,
                        qkv=w.qkv, bias=w.bias, seed=seed, device=device)
    out["bias_transpose"] = w.bias_transpose
    return out


# ---------------------------------------------------------------- SwiGLU transition

@dataclass(frozen=True)
class TransitionWorkload:
    """Layer norm, two expansions to n*C hidden units, silu(a)*b, projection back to C."""
    name: str
    a: int
    b: int
    channels: int
    expansion: int
    dtype: str
    desc: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def tokens(self) -> int:
        return self.a * self.b

    @property
    def hidden(self) -> int:
        return self.expansion * self.channels

    def flops_fwd(self) -> float:
        """Three T x C x nC products (two expansions, one projection)."""
        return 2.0 * 3 * self.tokens * self.channels * self.hidden

    def flops_fwd_bwd(self) -> float:
        """Forward 3, backward 6 products (dh, dy from da and db, and the three weight
        gradients); the a, b recompute of the backward is not counted."""
        return 2.0 * 9 * self.tokens * self.channels * self.hidden


TRANSITION_WORKLOADS = {
    "pair_transition_fp32_n48": TransitionWorkload(
        "pair_transition_fp32_n48", 48, 48, 128, 4, "fp32", "pair tensor N=48, C=128, n=4, fp32"),
    # The pair transition at the headline crop (N=384, C=128, 512 hidden units).
    "pair_transition_bf16_n384": TransitionWorkload(
        "pair_transition_bf16_n384", 384, 384, 128, 4, "bf16", "pair tensor N=384, C=128, n=4, bf16"),
    "msa_transition_bf16_s512_n384": TransitionWorkload(
        "msa_transition_bf16_s512_n384", 512, 384, 64, 4, "bf16", "MSA tensor S=512 N=384, C=64, n=4, bf16"),
}


def generate_transition(a: int, b: int, channels: int, expansion: int, *, dtype=torch.bfloat16, seed: int = 0,
                        device="cpu"):
    """Draw one seeded input set for the transition.

    Draw order with one torch CPU generator: x, per-token scale, per-token offset,
    gamma, beta, w_a, w_b, w_out, dout.  x, gamma and beta as for the projections;
    w_a, w_b ~ N(0, 1/C) and w_out ~ N(0, 1/(n*C)) (fan-in scaling) in the compute
    dtype; dout ~ N(0, 1)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    hidden = expansion * channels
    x = torch.randn((a, b, channels), generator=gen, dtype=torch.float32)
    scale = torch.exp(0.5 * torch.randn((a, b, 1), generator=gen, dtype=torch.float32))
    offset = torch.randn((a, b, 1), generator=gen, dtype=torch.float32)
    x = x * scale + offset
    gamma = 1.0 + 0.1 * torch.randn(channels, generator=gen, dtype=torch.float32)
    beta = 0.1 * torch.randn(channels, generator=gen, dtype=torch.float32)
    w_a = torch.randn((hidden, channels), generator=gen, dtype=torch.float32) / math.sqrt(channels)
    w_b = torch.randn((hidden, channels), generator=gen, dtype=torch.float32) / math.sqrt(channels)
    w_out = torch.randn((channels, hidden), generator=gen, dtype=torch.float32) / math.sqrt(hidden)
    dout = torch.randn((a, b, channels), generator=gen, dtype=torch.float32)

    def cast(t, dt=dtype):
        return t.to(dt).to(device).contiguous()

    return {"x": cast(x), "gamma": cast(gamma, torch.float32), "beta": cast(beta, torch.float32),
            "w_a": cast(w_a), "w_b": cast(w_b), "w_out": cast(w_out), "dout": cast(dout), "eps": 1e-5,
            "expansion": expansion}


def generate_transition_workload(w: TransitionWorkload, *, seed: int = 0, device="cpu"):
    return generate_transition(w.a, w.b, w.channels, w.expansion, dtype=w.torch_dtype, seed=seed, device=device)
