"""The forward entry point that allocates nothing (evoattn_fwd_noalloc), called
through the C ABI with every tensor allocated beforehand: its results equal those
of evoattn_fwd (same kernels, its scratch a static device array instead of a
caller's workspace) on two calls in a row, the second with a smaller problem, so
that the second runs on scratch that still holds the first call's contents."""
import ctypes
import math

import pytest
import torch

from af3_attention_amd import _lib
from workloads import generate

pytestmark = pytest.mark.gpu

_DT = {torch.float32: 0, torch.bfloat16: 1}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dims(q, transpose):
    if transpose:
        N, R, H, D = q.shape
    else:
        R, N, H, D = q.shape
    return R, N, H, D


def _inputs(R, N, H, D, dtype, transpose, seed):
    inp = generate(R, N, H, D, dtype=dtype, transpose=transpose, bias_std=math.sqrt(2),
                   mask_kind="tail_uniform", mask_frac=0.15, seed=seed)
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _noalloc(lib, g, transpose, o, lse):
    R, N, H, D = _dims(g["q"], transpose)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.evoattn_fwd_noalloc(R, N, H, D, _DT[g["q"].dtype], int(transpose), _p(g["q"]), _p(g["k"]),
                                   _p(g["v"]), _p(g["bias"]), _p(g["mask"]), _p(o), _p(lse), stream)


def _with_workspace(lib, g, transpose):
    R, N, H, D = _dims(g["q"], transpose)
    dt = _DT[g["q"].dtype]
    o = torch.empty_like(g["q"])
    lse = torch.empty((R, H, N), dtype=torch.float32, device="cuda")
    ws_bytes = int(lib.evoattn_fwd_workspace_bytes(R, N, H, D, dt))
    ws = torch.full((max(ws_bytes, 1),), 0x7f, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.evoattn_fwd(R, N, H, D, dt, int(transpose), _p(g["q"]), _p(g["k"]), _p(g["v"]), _p(g["bias"]),
                         _p(g["mask"]), _p(o), _p(lse), _p(ws), ws_bytes, stream)
    assert st == 0, lib.evoattn_last_error_detail().decode()
    return o, lse


@pytest.mark.parametrize("dtype,transpose", [(torch.bfloat16, 0), (torch.bfloat16, 1), (torch.float32, 0)])
def test_noalloc_matches_workspace_entry_point(dtype, transpose):
    lib = _lib.load()
    # A large problem, then a smaller one on the scratch the first one left behind.
    cases = [(40, 200, 4, 32, 11), (9, 70, 2, 16, 12)] if dtype == torch.bfloat16 else \
        [(20, 100, 4, 32, 13), (5, 33, 2, 8, 14)]
    for R, N, H, D, seed in cases:
        print(f"\n[no-alloc] dtype={dtype} t={transpose} R={R} N={N} H={H} D={D}", flush=True)
        g = _inputs(R, N, H, D, dtype, transpose, seed)
        ref_o, ref_lse = _with_workspace(lib, g, transpose)
        o = torch.empty_like(g["q"])
        lse = torch.empty((R, H, N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        st = _noalloc(lib, g, transpose, o, lse)
        assert st == 0, lib.evoattn_last_error_detail().decode()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), float((o.float() - ref_o.float()).abs().max())
        assert torch.equal(lse, ref_lse), float((lse - ref_lse).abs().max())


def test_noalloc_rejects_problems_beyond_its_scratch():
    lib = _lib.load()
    cap = 32 << 20
    R, N, H, D = 1536, 1536, 4, 32
    need = int(lib.evoattn_fwd_workspace_bytes(R, N, H, D, 1))
    assert need > cap
    x = torch.zeros(1, device="cuda")
    st = lib.evoattn_fwd_noalloc(R, N, H, D, 1, 0, _p(x), _p(x), _p(x), None, None, _p(x), _p(x), None)
    assert st == 3  # EVOATTN_ERR_WORKSPACE, before anything is launched
    assert "at most" in lib.evoattn_last_error_detail().decode()
