#!/usr/bin/env python3
"""Throughput of pair-biased 3D attention (forward + backward) on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
evoattn_fwd (O, lse) followed by evoattn_bwd (dQ, dK, dV, dBias), with every
input already resident in HBM.  The default workload is starting-node
triangle attention at an AF3 training crop: N = 384 rows and positions, H = 4
heads, d = 32, bf16 storage with fp32 accumulation, bias ~ N(0, 2), tail key
mask.  Flops are counted as 4*R*N^2*H*d for the forward and 10*R*N^2*H*d for
the backward (five N x N x d contractions, one of them the recompute of
Q K^T).

Prints one JSON line.  Besides the throughput it reports
  roofline      the kernel with the largest share of the step: algorithmic
                flops (or bytes) per launch divided by its mean launch time,
                measured with HIP events recorded by the library on the launch
                stream during a second timed pass of the same steps (the first
                pass, which gives the throughput, runs without them), against
                the MI355X peak; traffic is the HBM bytes per launch from the
                committed counter record, while the kernel's sources match it;
  cpu_baseline  the fp64 CPU oracle timed on this host's cores on a bounded
                sample of rows of the same workload (skip with --no-cpu-baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "fwd+bwd TFLOP/s (% bf16 MFMA peak), triangle attn N=384 H=4 d=32"
UNIT = "TFLOP/s"

# MI355X published peaks.
PEAK_BF16_MFMA_TFLOPS = 2500.0   # dense bf16 matrix
PEAK_FP32_VECTOR_TFLOPS = 157.3  # fp32 vector ALU
PEAK_HBM_GBS = 8000.0
# Vector ALU issue peak for the non-packed 32-bit operations these kernels use:
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane operations per second (the
# 157.3 TFLOP/s figure counts an FMA as two flops and two lanes per packed
# instruction; packed fp32 instructions are not used here).
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12

# Algorithmic work per launch of each kernel, in multiples of R*N^2*H*d flops
# (score elements times head_dim), with the unit that bounds it.
KERNEL_FLOP_FACTOR = {
    "fwd_mfma": (4.0, "mfma"),
    "bwd_mfma": (10.0, "mfma"),
    "bwd_fused_mfma": (10.0, "mfma"),
    "bwd_dkdv_mfma": (8.0, "mfma"),
    "bwd_dq_mfma": (6.0, "mfma"),
    "bwd_dbias_mfma": (4.0, "mfma"),
    "fwd_vector": (4.0, "alu"),
    "bwd_dq_vector": (6.0, "alu"),
    "bwd_dkdv_vector": (8.0, "alu"),
    "bwd_dbias_vector": (4.0, "alu"),
}

# Vector-ALU work each bf16 kernel needs per score element, in 32-bit lane
# operations: the scale (or the FMA that also subtracts the reference point), the
# exp2, the running sum (forward) or dS = P dP (backward) or the dBias
# accumulation, and the packing of P and dS to bf16 (one cvt_pk per two values).
KERNEL_VALU_OPS = {
    "fwd_mfma": 3.5,        # fma, exp2, add, cvt/2
    "bwd_fused_mfma": 4.0,  # mul, exp2, mul, cvt/2 for P and for dS
    "bwd_dkdv_mfma": 4.0,
    "bwd_dq_mfma": 3.5,     # mul, exp2, mul, cvt/2 for dS
    "bwd_dbias_mfma": 3.0,  # mul, exp2, fma
}


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "af3_attention_amd", "csrc")
# The source files each timed kernel is compiled from: a traffic record counts only
# while these are unchanged since its counters were taken.
COMMON_SOURCES = ["evoattn_internal.h", "mfma_common.h", "pipe_common.h"]
KERNEL_SOURCES = {
    "fwd_mfma": ["kernels_mfma_fwd.hip", "kernels_fwd_pp.hip", "kernels_bias_prep.hip", "dma_common.h"],
    "bwd_fused_mfma": ["kernels_bwd_fused.hip"],
    "bwd_dkdv_mfma": ["kernels_bwd_dkdv.hip"],
    "bwd_dq_mfma": ["kernels_bwd_dq.hip"],
    "bwd_dbias_mfma": ["kernels_bwd_dbias.hip"],
    "ln_proj_fwd": ["kernels_ln_proj.hip", "proj_common.h"],
    "ln_proj_bwd_dx": ["kernels_ln_proj_bwd.hip", "proj_common.h"],
    "ln_proj_bwd_mpart": ["kernels_ln_proj_bwd.hip", "proj_common.h"],
    "transition_fwd": ["kernels_transition.hip", "transition_common.h", "proj_common.h"],
    "transition_bwd_dx": ["kernels_transition_bwd.hip", "transition_common.h", "proj_common.h"],
    "transition_bwd_wpart": ["kernels_transition_bwd.hip", "transition_common.h", "proj_common.h"],
}


def sources_digest(kernel):
    """sha256 (first 16 hex digits) over the kernel's source files, or None."""
    import hashlib

    if kernel not in KERNEL_SOURCES:
        return None
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch (fetch + write) from the committed counter record.

    profiles/hbm_traffic_<workload>.md holds one line per kernel,
    "record: kernel=<name> fetch_bytes=<B> write_bytes=<B> sources=<digest>",
    written from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) scaled by
    the copy calibration.  Returns None when there is no record for the kernel or
    its sources have changed since.
    """
    path = os.path.join(HERE, "profiles", f"hbm_traffic_{workload}.md")
    digest = sources_digest(kernel)
    if digest is None or not os.path.exists(path):
        return None
    for line in open(path):
        if not line.startswith("record:"):
            continue
        kv = dict(x.split("=", 1) for x in line[len("record:"):].split())
        if kv.get("kernel") == kernel and kv.get("sources") == digest:
            return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def warm_up(step, args, sync):
    """The --warmup untimed steps, then more until --min-warmup-ms of wall time has
    passed.  Returns (extra steps, warm-up seconds)."""
    t0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    sync()
    extra = 0
    while (time.perf_counter() - t0) * 1e3 < args.min_warmup_ms:
        for _ in range(5):
            step()
        sync()
        extra += 5
    return extra, time.perf_counter() - t0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (the GPU clocks take some tens of ms to settle)")
    ap.add_argument("--min-warmup-ms", type=float, default=300.0,
                    help="after the --warmup steps, keep running untimed steps until this much wall time of "
                         "warm-up has passed (the clocks of a GPU that was idle ramp up over the first few "
                         "hundred ms of work); the extra steps are reported in the JSON line")
    ap.add_argument("--workload", default="tri_start_bf16_n384",
                    help="an attention workload, a layer norm + projection workload "
                         "(pair_proj_bf16_n384, pair_proj_end_bf16_n768, msa_proj_bf16_s512_n384) or a SwiGLU "
                         "transition workload (pair_transition_bf16_n384, msa_transition_bf16_s512_n384): the "
                         "latter two print their step's own line")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 256 MiB device copy three times "
                         "(the reference kernel that scales HBM byte counters)")
    ap.add_argument("--memory-curve", action="store_true",
                    help="instead of the throughput line: peak extra HBM of one fwd+bwd at N = 64 .. 2048 "
                         "(R = N, H = 4, d = 32, bf16), beside a materialised fp32 torch reference until it "
                         "runs out of memory")
    ap.add_argument("--no-unfused", action="store_true",
                    help="projection workloads: skip the unfused torch layer_norm + mm pipeline timed beside")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the second pass with per-kernel HIP events (no roofline)")
    return ap.parse_args()


def cpu_baseline(w, inp, target_s):
    """Time the fp64 oracle (fwd + bwd) on a sample of rows sized to ~target_s seconds."""
    import numpy as np
    import oracle

    threads = len(os.sched_getaffinity(0))
    used = oracle.set_threads(threads)
    to64 = lambda t: None if t is None else t.detach().cpu().double().numpy()
    q, k, v, b, m, do = (to64(inp[x]) for x in ("q", "k", "v", "bias", "mask", "dout"))
    t = inp["transpose"]

    def run(rows):
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, b, m, t, rows=rows)
        oracle.bwd(q, k, v, b, m, do, t, rows=rows)
        return time.perf_counter() - t0

    # Size the sample from a one-row probe, then once more from the first sample
    # if that fell well short of the target (the probe carries start-up costs).
    probe = run([0])
    nrows, secs = 1, probe
    for _ in range(2):
        if secs >= 0.6 * target_s or nrows >= w.rows:
            break
        nrows = int(max(1, min(w.rows, nrows * target_s / max(secs, 1e-6))))
        secs = run(list(range(nrows)))
    # A host fast enough to finish every row early repeats the whole workload.
    reps = 1
    if nrows >= w.rows and secs < 0.6 * target_s:
        reps = int(min(8, max(2, round(target_s / max(secs, 1e-6)))))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(list(range(nrows)))
        secs = time.perf_counter() - t0
    per_row_flops = 14.0 * w.n * w.n * w.heads * w.head_dim
    value = per_row_flops * nrows * reps / secs / 1e12
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": value, "unit": UNIT, "cores": used, "kind": "oracle",
        "sample": f"rows 0..{nrows - 1} of {w.rows} of {w.name} (fwd+bwd, fp64)"
                  + (f" x {reps} passes" if reps > 1 else "") + f", {secs:.2f} s",
        "seconds": secs, "cpu_model": cpu_model,
    }


def memory_curve():
    """Peak HBM of one fwd + bwd versus N, for this library and a materialised reference.

    The library keeps O(R*H*N + H*N^2) bytes besides its inputs and outputs.  The
    reference forms the [R,H,N,N] scores, probabilities and their gradients in fp32
    with torch autograd until it runs out of memory.  It runs in fp32 because the
    backward of a bf16 batched product makes torch issue batched products whose
    right operand is a transposed view, and those have faulted GPUs of this kind;
    a bf16 reference would hold the same tensors at half the bytes.  The last record
    is the long-sequence case run back to back: the starting-node and the
    ending-node forward with both outputs and lse kept, then both backward passes.
    """
    import torch
    import af3_attention_amd as ea
    from workloads import generate

    dev = torch.device("cuda:0")
    out = []
    reference_alive = True
    for n in (64, 128, 256, 384, 512, 768, 1024, 1536, 2048):
        inp = generate(n, n, 4, 32, dtype=torch.bfloat16, bias_std=2 ** 0.5, mask_kind="tail_fixed",
                       mask_frac=0.05, seed=0)
        g = {x: (None if inp[x] is None else inp[x].to(dev)) for x in ("q", "k", "v", "bias", "mask", "dout")}
        del inp
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        o, lse = ea.evoattn_fwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], False)
        grads = ea.evoattn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, lse, g["dout"], False)
        torch.cuda.synchronize()
        fused = torch.cuda.max_memory_allocated(dev) - base
        del o, lse, grads
        row = {"n": n, "rows": n, "inputs_bytes": base, "fused_peak_extra_bytes": fused}
        if reference_alive:
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats(dev)
            try:
                q, k, v = (g[x].float().permute(0, 2, 1, 3).contiguous().requires_grad_() for x in ("q", "k", "v"))
                bias = g["bias"].float().requires_grad_()
                s = torch.matmul(q, k.transpose(-1, -2).contiguous()) / 32 ** 0.5 + bias[None] \
                    + g["mask"][:, None, None, :]
                o_ref = torch.matmul(torch.softmax(s, dim=-1), v)
                o_ref.backward(g["dout"].float().permute(0, 2, 1, 3).contiguous())
                torch.cuda.synchronize()
                row["reference_peak_extra_bytes"] = torch.cuda.max_memory_allocated(dev) - base
            except torch.cuda.OutOfMemoryError:
                row["reference_peak_extra_bytes"] = "out of memory"
                reference_alive = False
            q = k = v = bias = s = o_ref = None
            torch.cuda.empty_cache()
        else:
            row["reference_peak_extra_bytes"] = "not run (out of memory at a smaller N)"
        out.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del g
    # N = 1536, both variants back to back with both forward results live.
    n = 1536
    gs = []
    for t in (0, 1):
        inp = generate(n, n, 4, 32, dtype=torch.bfloat16, transpose=t, bias_std=2 ** 0.5, mask_kind="tail_fixed",
                       mask_frac=0.05, seed=t)
        gs.append({x: (None if inp[x] is None else inp[x].to(dev)) for x in ("q", "k", "v", "bias", "mask", "dout")})
        del inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    fwd_out = [ea.evoattn_fwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], bool(t)) for t, g in enumerate(gs)]
    grads = [ea.evoattn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, lse, g["dout"], bool(t))
             for t, (g, (o, lse)) in enumerate(zip(gs, fwd_out))]
    torch.cuda.synchronize()
    back_to_back = {"n": n, "rows": n, "variants": [0, 1], "inputs_bytes": base,
                    "fused_peak_extra_bytes": torch.cuda.max_memory_allocated(dev) - base}
    print(json.dumps(back_to_back), file=sys.stderr, flush=True)
    del fwd_out, grads, gs
    total = torch.cuda.get_device_properties(dev).total_memory
    print(json.dumps({"memory_curve": out, "back_to_back_n1536": back_to_back, "device_memory_bytes": total,
                      "dtype": "bf16", "config": {"heads": 4, "head_dim": 32, "mask": "tail 5%"}}), flush=True)


def copy_calibration(dev):
    """An elementwise kernel that reads and writes exactly 256 MiB each (negation of a
    contiguous fp32 tensor), run three times: its FETCH_SIZE and WRITE_SIZE readings
    give the factor between counter bytes and true HBM bytes."""
    import torch

    nbytes = 256 << 20
    src = torch.randn(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"kernel": "torch.neg fp32", "read_bytes": nbytes, "write_bytes": nbytes, "launches": 3}


# ---------------------------------------------------------------- layer norm + projections

PROJ_METRIC = "layer norm + q/k/v/bias projections fwd+bwd, effective HBM GB/s"


def proj_bytes(w, es):
    """Algorithmic HBM bytes of the projection step and of each kernel launch.

    The step's bytes are what a single fused pass must move: forward x in, q, k, v,
    bias and the statistics out; backward x, the upstream gradients (dbias in fp32)
    and the statistics in, dx out; weights and their gradients once each."""
    T, C, H = w.tokens, w.channels, w.heads
    n_qkv = 3 * H * w.head_dim if w.qkv else 0
    nb = H if w.bias else 0
    n_out = n_qkv + nb
    weights = n_out * C * es + 2 * C * 4
    fwd = T * C * es + T * n_qkv * es + T * nb * es + T * 8 + weights
    grads_in = T * n_qkv * es + T * nb * 4
    hb = -(-nb // 16) * 16
    gb = T * hb * 2  # the bias gradient in token order, bf16, written once and read by dx and mpart
    bwd_dx = T * C * es + T * n_qkv * es + gb + T * 8 + T * C * es + weights
    chunks = -(-T // 128)
    ranges = min(64, chunks)
    per = -(-chunks // ranges)
    ranges = -(-chunks // per)
    po = -(-n_out // 32) * 32
    partial = ranges * po * (C + 1) * 4
    bwd_mpart = T * C * es + T * n_qkv * es + gb + T * 8 + partial
    step = fwd + (T * C * es + grads_in + T * 8 + T * C * es) + weights + n_out * C * 4 + 2 * C * 4
    return step, {"ln_proj_fwd": fwd, "ln_proj_bwd_dx": bwd_dx, "ln_proj_bwd_mpart": bwd_mpart,
                  "ln_proj_bwd_finalize": partial + 3 * n_out * C * 4, "ln_proj_bwd_bias_tokens": T * nb * 4 + gb}


def proj_cpu_baseline(w, inp, target_s):
    """The fp64 oracle (fwd + bwd) on an s x s token sub-grid sized to ~target_s seconds."""
    import numpy as np
    import oracle

    threads = len(os.sched_getaffinity(0))
    f = lambda t: None if t is None else t.detach().cpu().double().numpy()
    H, D, bt = w.heads, w.head_dim, w.bias_transpose

    def run(s):
        sub = lambda t: None if t is None else t[:s, :s]
        x = f(sub(inp["x"]))
        t0 = time.perf_counter()
        oracle.ln_proj_fwd(x, f(inp["gamma"]), f(inp["beta"]), inp["eps"], f(inp["w_qkv"]), f(inp["w_bias"]),
                           H, D, bt)
        oracle.ln_proj_bwd(x, f(inp["gamma"]), f(inp["beta"]), inp["eps"], f(inp["w_qkv"]), f(inp["w_bias"]),
                           H, D, bt, f(sub(inp["dq"])), f(sub(inp["dk"])), f(sub(inp["dv"])),
                           None if inp["dbias"] is None else f(inp["dbias"][:, :s, :s]))
        return time.perf_counter() - t0

    side = min(w.a, w.b)
    s, secs = 16, run(16)
    for _ in range(3):
        if secs >= 0.6 * target_s or s >= side:
            break
        s = int(min(side, max(s + 1, s * (target_s / max(secs, 1e-6)) ** 0.5)))
        secs = run(s)
    # A host that finishes the whole grid early repeats it.
    reps = 1
    if s >= side and secs < 0.6 * target_s:
        reps = int(min(60, max(2, round(target_s / max(secs, 1e-6)))))
        secs = sum(run(s) for _ in range(reps))
    sample = type(w)(w.name, s, s, w.channels, w.heads, w.head_dim, w.dtype, w.qkv, w.bias, w.bias_transpose)
    step_bytes, _ = proj_bytes(sample, 2 if w.dtype == "bf16" else 4)
    return {"value": step_bytes * reps / secs / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{s} x {s} token sub-grid of {w.name} (fwd+bwd, fp64)"
                      + (f" x {reps} passes" if reps > 1 else "") + f", {secs:.2f} s", "seconds": secs}


def proj_main(args, w):
    import torch
    import af3_attention_amd as ea
    from af3_attention_amd import _lib
    from workloads import generate_proj_workload

    dev = torch.device("cuda:0")
    es = 2 if w.dtype == "bf16" else 4
    inp_cpu = generate_proj_workload(w, seed=args.seed)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp_cpu.items()}
    H, D, bt = w.heads, w.head_dim, w.bias_transpose
    ws = torch.empty(ea.ln_proj_bwd_workspace_bytes(w.a, w.b, w.channels, H, D, w.torch_dtype, w.qkv, w.bias),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        fw = ea.ln_proj_fwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], heads=H, head_dim=D,
                            bias_transpose=bt, eps=g["eps"])
        ea.ln_proj_bwd(g["x"], g["gamma"], g["beta"], g["w_qkv"], g["w_bias"], fw["mean"], fw["rstd"], g["dq"],
                       g["dk"], g["dv"], g["dbias"], heads=H, head_dim=D, bias_transpose=bt, workspace=ws)

    stream = torch.cuda.current_stream(dev)

    def timed(fn, kernel_timing=False):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _lib.timing_collect()
        _lib.timing_enable(kernel_timing)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        _lib.timing_enable(False)
        return start.elapsed_time(stop) / args.steps, _lib.timing_collect()

    warm_extra, warm_s = warm_up(step, args, torch.cuda.synchronize)
    base_mem = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ms, _ = timed(step)
    peak_fused = torch.cuda.max_memory_allocated(dev) - base_mem
    kernels = {}
    if not args.no_kernel_timing:
        _, kernels = timed(step, True)
    step_bytes, kbytes = proj_bytes(w, es)
    value = step_bytes / (ms * 1e-3) / 1e9

    roofline = None
    if kernels:
        name, (count, tot) = max(kernels.items(), key=lambda kv: kv[1][1])
        avg_ms = tot / count
        if name in kbytes:
            achieved = kbytes[name] / (avg_ms * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": achieved / PEAK_HBM_GBS, "traffic": recorded_traffic(name, w.name),
                        "kernel": name, "avg_launch_ms": avg_ms, "launches": count,
                        "algorithmic_bytes": kbytes[name]}

    unfused = None
    if not args.no_unfused:
        unfused = proj_unfused(w, g, args, stream)

    cpu = None if args.no_cpu_baseline else proj_cpu_baseline(w, inp_cpu, args.cpu_seconds)
    line = {
        "metric": PROJ_METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_extra_steps": warm_extra, "warmup_s": round(warm_s, 3), "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "a": w.a, "b": w.b, "channels": w.channels, "heads": H, "head_dim": D,
                   "qkv": w.qkv, "bias": w.bias, "bias_transpose": bt, "seed": args.seed},
        "tokens_per_s": w.tokens / (ms * 1e-3),
        "step_algorithmic_bytes": step_bytes,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "unfused_torch": unfused,
        "kernels_ms_per_step": {k: tot / args.steps for k, (c, tot) in kernels.items()},
        "peak_hbm_extra_bytes": int(peak_fused + ws.numel()),  # the workspace is allocated up front
    }
    if args.copy_calibration:
        line["copy_calibration"] = copy_calibration(dev)
    print(json.dumps(line), flush=True)


def proj_unfused(w, g, args, stream):
    """The same step as separate torch kernels (bf16 layer norm, then one mm per
    projection; backward by mm and the layer-norm backward), which materialise
    the normalised tensor and its gradient in HBM.  Only 2-D products are used."""
    import torch

    T, C, H = w.tokens, w.channels, w.heads
    hd = H * w.head_dim
    dt = w.torch_dtype
    dev = g["x"].device
    x2 = g["x"].view(T, C)
    gam, bet = g["gamma"].to(dt), g["beta"].to(dt)
    ws = []
    if w.qkv:
        ws += [g["w_qkv"][i * hd:(i + 1) * hd].contiguous() for i in range(3)]
    if w.bias:
        ws.append(g["w_bias"].contiguous())
    wts = [x.t().contiguous() for x in ws]
    grads = []
    if w.qkv:
        grads += [g[n].view(T, hd) for n in ("dq", "dk", "dv")]
    if w.bias:
        db = g["dbias"].transpose(1, 2) if w.bias_transpose else g["dbias"]
        grads.append(db.reshape(H, T).t().contiguous().to(dt))

    def step():
        y, mean, rstd = torch.native_layer_norm(x2, (C,), gam, bet, g["eps"])
        outs = [torch.mm(y, wt) for wt in wts]
        if w.bias:
            b = outs[-1].t().contiguous()
            if w.bias_transpose:
                b = b.view(H, w.a, w.b).transpose(1, 2).contiguous()
        dy = torch.mm(grads[0], ws[0])
        for gr, wm in zip(grads[1:], ws[1:]):
            dy.addmm_(gr, wm)
        dws = [torch.mm(gr.t(), y) for gr in grads]
        torch.ops.aten.native_layer_norm_backward(dy, x2, (C,), mean, rstd, gam, bet, [True, True, True])
        return dws

    for _ in range(max(5, args.warmup // 10)):
        step()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    return {"ms_per_step": ms, "peak_hbm_extra_bytes": int(torch.cuda.max_memory_allocated(dev) - base),
            "ops": "native_layer_norm, mm per projection, addmm, mm (weight grads), native_layer_norm_backward"}


# ---------------------------------------------------------------- SwiGLU transition

TRANS_METRIC = "SwiGLU transition fwd+bwd TFLOP/s (9 T*C*nC products, recompute not counted)"

# Products of shape T x C x nC each kernel launch performs (its own algorithm,
# recomputation included), times 2 flops.
TRANS_KERNEL_PRODUCTS = {"transition_fwd": 3, "transition_bwd_dx": 5, "transition_bwd_wpart": 6}


def transition_cpu_baseline(w, inp, target_s):
    """The fp64 oracle (fwd + bwd) on an s x s token sub-grid sized to ~target_s seconds."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    f = lambda t: t.detach().cpu().double().numpy()
    wts = [f(inp[n]) for n in ("gamma", "beta")] + [inp["eps"]] + [f(inp[n]) for n in ("w_a", "w_b", "w_out")]

    def run(s):
        x, do = f(inp["x"][:s, :s]), f(inp["dout"][:s, :s])
        t0 = time.perf_counter()
        oracle.transition_fwd(x, *wts)
        oracle.transition_bwd(x, *wts, do)
        return time.perf_counter() - t0

    side = min(w.a, w.b)
    s, secs = 8, run(8)
    for _ in range(3):
        if secs >= 0.6 * target_s or s >= side:
            break
        s = int(min(side, max(s + 1, s * (target_s / max(secs, 1e-6)) ** 0.5)))
        secs = run(s)
    reps = 1
    if s >= side and secs < 0.6 * target_s:
        reps = int(min(60, max(2, round(target_s / max(secs, 1e-6)))))
        secs = sum(run(s) for _ in range(reps))
    flops = 2.0 * 9 * s * s * w.channels * w.hidden * reps
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{s} x {s} token sub-grid of {w.name} (fwd+bwd, fp64)"
                      + (f" x {reps} passes" if reps > 1 else "") + f", {secs:.2f} s", "seconds": secs}


def transition_unfused(w, g, args, stream):
    """The same step as separate torch kernels in bf16 (layer norm, one mm per
    product, elementwise gate and its derivative, layer-norm backward), which
    materialise y, a, b, h and their gradients in HBM.  Only 2-D products."""
    import torch

    T, C, Hd = w.tokens, w.channels, w.hidden
    dt = w.torch_dtype
    dev = g["x"].device
    x2, do2 = g["x"].view(T, C), g["dout"].view(T, C)
    gam, bet = g["gamma"].to(dt), g["beta"].to(dt)
    wa, wb, wo = g["w_a"], g["w_b"], g["w_out"]
    wat, wbt, wot = wa.t().contiguous(), wb.t().contiguous(), wo.t().contiguous()

    def step():
        y, mean, rstd = torch.native_layer_norm(x2, (C,), gam, bet, g["eps"])
        a = torch.mm(y, wat)
        b = torch.mm(y, wbt)
        sa = torch.nn.functional.silu(a)
        h = sa * b
        torch.mm(h, wot)
        dh = torch.mm(do2, wo)
        sg = torch.sigmoid(a)
        da = dh * b * (sg * (1 + a * (1 - sg)))
        db = dh * sa
        dy = torch.mm(da, wa)
        dy.addmm_(db, wb)
        torch.mm(do2.t(), h)
        torch.mm(da.t(), y)
        torch.mm(db.t(), y)
        torch.ops.aten.native_layer_norm_backward(dy, x2, (C,), mean, rstd, gam, bet, [True, True, True])

    for _ in range(max(5, args.warmup // 10)):
        step()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    return {"ms_per_step": ms, "tflops": 2.0 * 9 * T * C * Hd / (ms * 1e-3) / 1e12,
            "peak_hbm_extra_bytes": int(torch.cuda.max_memory_allocated(dev) - base),
            "ops": "native_layer_norm, mm per product, silu/sigmoid elementwise, native_layer_norm_backward"}


def transition_main(args, w):
    import torch
    import af3_attention_amd as ea
    from af3_attention_amd import _lib
    from workloads import generate_transition_workload

    dev = torch.device("cuda:0")
    inp_cpu = generate_transition_workload(w, seed=args.seed)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp_cpu.items()}
    ws = torch.empty(ea.transition_bwd_workspace_bytes(w.a, w.b, w.channels, w.expansion), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def step():
        fw = ea.transition_fwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], eps=g["eps"])
        ea.transition_bwd(g["x"], g["gamma"], g["beta"], g["w_a"], g["w_b"], g["w_out"], fw["mean"], fw["rstd"],
                          g["dout"], workspace=ws)

    stream = torch.cuda.current_stream(dev)

    def timed(fn, kernel_timing=False):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _lib.timing_collect()
        _lib.timing_enable(kernel_timing)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        _lib.timing_enable(False)
        return start.elapsed_time(stop) / args.steps, _lib.timing_collect()

    warm_extra, warm_s = warm_up(step, args, torch.cuda.synchronize)
    base_mem = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ms, _ = timed(step)
    peak_fused = torch.cuda.max_memory_allocated(dev) - base_mem
    kernels = {}
    if not args.no_kernel_timing:
        _, kernels = timed(step, True)
    unit_flops = 2.0 * w.tokens * w.channels * w.hidden
    value = 9 * unit_flops / (ms * 1e-3) / 1e12
    roofline = None
    if kernels:
        name, (count, tot) = max(kernels.items(), key=lambda kv: kv[1][1])
        avg_ms = tot / count
        if name in TRANS_KERNEL_PRODUCTS:
            achieved = TRANS_KERNEL_PRODUCTS[name] * unit_flops / (avg_ms * 1e-3) / 1e12
            roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                        "frac": achieved / PEAK_BF16_MFMA_TFLOPS, "traffic": recorded_traffic(name, w.name),
                        "kernel": name, "avg_launch_ms": avg_ms, "launches": count,
                        "algorithmic_flops": TRANS_KERNEL_PRODUCTS[name] * unit_flops}
    unfused = None if args.no_unfused else transition_unfused(w, g, args, stream)
    cpu = None if args.no_cpu_baseline else transition_cpu_baseline(w, inp_cpu, args.cpu_seconds)
    line = {
        "metric": TRANS_METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_extra_steps": warm_extra, "warmup_s": round(warm_s, 3), "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "a": w.a, "b": w.b, "channels": w.channels, "expansion": w.expansion,
                   "seed": args.seed},
        "frac_of_bf16_peak": value / PEAK_BF16_MFMA_TFLOPS,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "unfused_torch": unfused,
        "kernels_ms_per_step": {k: tot / args.steps for k, (c, tot) in kernels.items()},
        "peak_hbm_extra_bytes": int(peak_fused + ws.numel()),  # the workspace is allocated up front
    }
    if args.copy_calibration:
        line["copy_calibration"] = copy_calibration(dev)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.memory_curve and args.gpus == 1:
        memory_curve()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    from workloads import PROJ_WORKLOADS, TRANSITION_WORKLOADS
    if args.workload in PROJ_WORKLOADS:
        proj_main(args, PROJ_WORKLOADS[args.workload])
        return
    if args.workload in TRANSITION_WORKLOADS:
        transition_main(args, TRANSITION_WORKLOADS[args.workload])
        return

    import torch
    import af3_attention_amd as ea
    from af3_attention_amd import _lib
    from workloads import WORKLOADS, generate_workload

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    variants = list(w.variants) if len(w.variants) > 1 else [w.transpose]
    inputs_cpu = [generate_workload(w, transpose=t, seed=args.seed + i) for i, t in enumerate(variants)]
    inputs = [{x: (v.to(dev) if torch.is_tensor(v) else v) for x, v in inp.items()} for inp in inputs_cpu]
    torch.cuda.synchronize()

    def step():
        saved = []
        for inp in inputs:
            o, lse = ea.evoattn_fwd(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], bool(inp["transpose"]))
            saved.append((o, lse))
        for inp, (o, lse) in reversed(list(zip(inputs, saved))):
            ea.evoattn_bwd(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], o, lse, inp["dout"],
                           bool(inp["transpose"]))

    warm_extra, warm_s = warm_up(step, args, torch.cuda.synchronize)
    torch.cuda.reset_peak_memory_stats(dev)
    base_mem = torch.cuda.memory_allocated(dev)

    stream = torch.cuda.current_stream(dev)

    def timed(kernel_timing):
        """Time exactly args.steps steps; returns (ms per step, per-kernel records)."""
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _lib.timing_collect()  # drop anything recorded before
        _lib.timing_enable(kernel_timing)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        _lib.timing_enable(False)
        return start.elapsed_time(stop) / args.steps, _lib.timing_collect()

    # The throughput pass runs without per-kernel events (each launch would gain
    # two event records, a few microseconds of gap); a second pass of the same
    # steps records them, for the roofline of the dominant kernel.
    ms_per_step, _ = timed(False)

    # Forward alone (the same inputs, the same number of steps).
    def fwd_only():
        for inp in inputs:
            ea.evoattn_fwd(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], bool(inp["transpose"]))

    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record(stream)
    for _ in range(args.steps):
        fwd_only()
    f1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / args.steps
    kernels = {}
    if not args.no_kernel_timing:
        events_ms_per_step, kernels = timed(True)
    peak_extra = torch.cuda.max_memory_allocated(dev) - base_mem

    flops_step = w.flops_fwd_bwd() * len(variants)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # Roofline of the dominant kernel: its matrix-core figure and, for the bf16
    # kernels, its vector-ALU figure; "roofline" is the nearer of the two roofs
    # (the larger fraction) and "roofline_other" the farther.
    dom = max(kernels.items(), key=lambda kv: kv[1][1]) if kernels else None
    roofline = roofline_other = None
    if dom:
        name, (count, tot) = dom
        avg_ms = tot / count
        factor, bound = KERNEL_FLOP_FACTOR.get(name, (None, None))
        launches_per_step = count / args.steps
        units = w.rows * w.n * w.n * w.heads * w.head_dim * len(variants) / launches_per_step
        if factor is not None:
            achieved = factor * units / (avg_ms * 1e-3) / 1e12
            peak = PEAK_BF16_MFMA_TFLOPS if bound == "mfma" else PEAK_FP32_VECTOR_TFLOPS
            roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                        "frac": achieved / peak, "traffic": recorded_traffic(name, w.name), "kernel": name,
                        "avg_launch_ms": avg_ms, "launches": count}
        if name in KERNEL_VALU_OPS and roofline is not None:
            scores = units / w.head_dim
            ach = KERNEL_VALU_OPS[name] * scores / (avg_ms * 1e-3) / 1e12
            valu = {"bound": "alu", "achieved": ach, "peak": PEAK_VALU_TOPS, "unit": "T lane-ops/s",
                    "frac": ach / PEAK_VALU_TOPS, "traffic": roofline["traffic"], "kernel": name,
                    "avg_launch_ms": avg_ms, "launches": count,
                    "ops_per_score": KERNEL_VALU_OPS[name]}
            if valu["frac"] > roofline["frac"]:
                roofline, roofline_other = valu, roofline
            else:
                roofline_other = valu

    calibration = copy_calibration(dev) if args.copy_calibration else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inputs_cpu[0], args.cpu_seconds)

    line = {
        "metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_extra_steps": warm_extra, "warmup_s": round(warm_s, 3), "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "n": w.n, "heads": w.heads, "head_dim": w.head_dim,
                   "transpose": variants, "mask": w.mask_kind, "seed": args.seed},
        "frac_of_bf16_peak": value / PEAK_BF16_MFMA_TFLOPS,
        "fwd_only": {"ms_per_step": fwd_ms, "tflops": w.flops_fwd() * len(variants) / (fwd_ms * 1e-3) / 1e12,
                     "frac_of_bf16_peak": w.flops_fwd() * len(variants) / (fwd_ms * 1e-3) / 1e12
                     / PEAK_BF16_MFMA_TFLOPS},
        "roofline": roofline,
        "roofline_other": roofline_other,
        "cpu_baseline": cpu,
        "kernels_ms_per_step": {k: tot / args.steps for k, (c, tot) in kernels.items()},
        "events_pass_ms_per_step": None if args.no_kernel_timing else events_ms_per_step,
        "peak_hbm_extra_bytes": int(peak_extra),
    }
    if calibration:
        line["copy_calibration"] = calibration
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
