"""CPU fp64 oracle for 3D attention with a broadcast pair bias (test infrastructure).

ORACLE -- TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
it imports nothing from the product path.

The arithmetic lives in `evo_oracle.c` (plain C, fp64, OpenMP, no fast-math,
no FMA contraction).  This module only builds that file with gcc and marshals
numpy float64 arrays into it.  Every function computes the plain definition of
attention with an additive pair bias and key mask, as described on the MegaFold
pages (gist.science technical summary, Methodik section 1 "EvoFlash-3D"): the
logits of each row are materialised in full and normalised with the ordinary
softmax.

Parity pins: every quantity returned here is pinned by the CPU test suite
(closed forms, invariants, central finite differences, a hand-derived worked
example and torch's fp64 scaled-dot-product attention with autograd).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "evo_oracle.c")
# EVO_ORACLE_SANITIZE=1 selects a build instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (gcc's runtimes, which the process must preload;
# tests/run_sanitizers.py does that).
_SANITIZE = os.environ.get("EVO_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "libevo_oracle_san.so" if _SANITIZE else "libevo_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile evo_oracle.c into libevo_oracle.so (gcc, -O2, OpenMP, IEEE semantics)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    san = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"] \
        if _SANITIZE else []
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *san, "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.evo_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.evo_oracle_set_threads.restype = ctypes.c_int
    lib.evo_oracle_fwd.argtypes = [i64, i64, i64, i64, ctypes.c_int, dp, dp, dp, dp, dp,
                                   ip, i64, dp, dp]
    lib.evo_oracle_fwd.restype = ctypes.c_int
    lib.evo_oracle_bwd.argtypes = [i64, i64, i64, i64, ctypes.c_int, dp, dp, dp, dp, dp, dp,
                                   ip, i64, dp, dp, dp, dp]
    lib.evo_oracle_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def set_threads(n: int) -> int:
    """Set the OpenMP thread count (n <= 0 leaves it unchanged); returns the count in use."""
    return int(_load().evo_oracle_set_threads(int(n)))


def _as_f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(q, transpose, mask, bias):
    a, b, H, D = q.shape
    R, N = (b, a) if transpose else (a, b)
    if bias is not None and bias.shape != (H, N, N):
        raise ValueError(f"bias shape {bias.shape} != {(H, N, N)}")
    if mask is not None and mask.shape != (R, N):
        raise ValueError(f"mask shape {mask.shape} != {(R, N)}")
    return R, N, H, D


def _rows_arg(rows, R):
    if rows is None:
        return None, 0, None
    r = np.ascontiguousarray(np.asarray(sorted(set(int(x) for x in rows)), dtype=np.int64))
    if r.size and (r[0] < 0 or r[-1] >= R):
        raise ValueError("row index out of range")
    return r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(r.size), r


def fwd(q, k, v, bias=None, mask=None, transpose=0, rows=None):
    """Returns (O, lse): O in q's physical layout, lse [R, H, N] (natural log), fp64.

    Rows not in `rows` (when given) are left as NaN in O and lse."""
    q, k, v, bias, mask = (_as_f64(t) for t in (q, k, v, bias, mask))
    R, N, H, D = _dims(q, transpose, mask, bias)
    o = np.full(q.shape, np.nan)
    lse = np.full((R, H, N), np.nan)
    rp, nr, _keep = _rows_arg(rows, R)
    rc = _load().evo_oracle_fwd(R, N, H, D, int(transpose), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(bias), _ptr(mask), rp, nr, _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"evo_oracle_fwd failed with code {rc}")
    return o, lse


def bwd(q, k, v, bias, mask, dout, transpose=0, rows=None):
    """Returns (dQ, dK, dV, dBias) in fp64 for the loss sum(O * dout).

    dBias [H, N, N] sums over the listed rows only (all rows by default), in
    increasing row order.  Gradients of unlisted rows are left as NaN."""
    q, k, v, bias, mask, dout = (_as_f64(t) for t in (q, k, v, bias, mask, dout))
    R, N, H, D = _dims(q, transpose, mask, bias)
    dq = np.full(q.shape, np.nan)
    dk = np.full(q.shape, np.nan)
    dv = np.full(q.shape, np.nan)
    dbias = np.zeros((H, N, N))
    rp, nr, _keep = _rows_arg(rows, R)
    rc = _load().evo_oracle_bwd(R, N, H, D, int(transpose), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(bias), _ptr(mask), _ptr(dout), rp, nr,
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias))
    if rc != 0:
        raise RuntimeError(f"evo_oracle_bwd failed with code {rc}")
    return dq, dk, dv, dbias


from .ln_proj import layer_norm, ln_proj_bwd, ln_proj_fwd  # noqa: E402,F401
from .transition import silu, silu_grad, transition_bwd, transition_fwd  # noqa: E402,F401
