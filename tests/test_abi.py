"""Boundary tests that need no GPU: the C header, the exported symbols and the
argument validation that runs before any launch."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from af3_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("evoattn.h", "evofusion.h")]

OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE = 0, 1, 2, 3, 4


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(evoattn_[a-z0-9_]+)\s*\(", text)))


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "evoattn.h"\n#include "evofusion.h"\n'
                   'int main(void){return evoattn_abi_version() == EVOATTN_ABI_VERSION ? 0 : 1;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                    str(src)], check=True)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (evoattn_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.evoattn_abi_version() == 1
    for code, name in ((OK, "EVOATTN_OK"), (INVALID, "EVOATTN_ERR_INVALID_ARGUMENT"),
                       (UNSUPPORTED, "EVOATTN_ERR_UNSUPPORTED"), (WORKSPACE, "EVOATTN_ERR_WORKSPACE"),
                       (DEVICE, "EVOATTN_ERR_DEVICE")):
        assert lib.evoattn_status_string(code).decode() == name
    assert lib.evoattn_status_string(99).decode() == "EVOATTN_UNKNOWN_STATUS"


def test_workspace_queries():
    lib = _lib.load()
    fws = lib.evoattn_fwd_workspace_bytes(384, 384, 4, 32, 1)
    assert fws % 256 == 0
    # one padded fp32 copy of the bias, 16 bytes per (row, key) of mask operands
    # and one int per row (each rounded up to 256 bytes) at most
    assert fws <= 4 * 512 * 512 * 4 + 384 * 384 * 16 + 384 * 4 + 3 * 256
    assert lib.evoattn_fwd_workspace_bytes(64, 64, 4, 32, 0) == 0   # fp32 path needs none
    ws = lib.evoattn_bwd_workspace_bytes(384, 384, 4, 32, 1)
    assert ws >= 384 * 4 * 384 * 4            # at least the per-row statistics
    assert ws % 256 == 0
    # O(R*H*N + H*N*N): far below one N^3 score tensor
    assert ws < 384 * 384 * 384 * 4 * 2 / 8
    assert lib.evoattn_bwd_workspace_bytes(0, 384, 4, 32, 1) == 0       # invalid -> 0
    assert lib.evoattn_bwd_workspace_bytes(8, 8, 4, 24, 1) == 0         # unsupported d -> 0


# Fake, aligned, never dereferenced addresses: every call below must fail validation
# before anything touches a device.
A = 1 << 20


def fwd(**kw):
    lib = _lib.load()
    args = dict(rows=4, n=8, heads=2, head_dim=32, dtype=1, transpose=0, q=A, k=A, v=A, bias=None, mask=None,
                o=A, lse=A, ws=A, ws_bytes=1 << 30)
    args.update(kw)
    return lib.evoattn_fwd(args["rows"], args["n"], args["heads"], args["head_dim"], args["dtype"],
                           args["transpose"], args["q"], args["k"], args["v"], args["bias"], args["mask"],
                           args["o"], args["lse"], args["ws"], args["ws_bytes"], None)


def bwd(**kw):
    lib = _lib.load()
    args = dict(rows=4, n=8, heads=2, head_dim=32, dtype=1, transpose=0, q=A, k=A, v=A, bias=None, mask=None,
                o=A, lse=A, dout=A, dq=A, dk=A, dv=A, dbias=None, ws=A, ws_bytes=1 << 30)
    args.update(kw)
    return lib.evoattn_bwd(args["rows"], args["n"], args["heads"], args["head_dim"], args["dtype"],
                           args["transpose"], args["q"], args["k"], args["v"], args["bias"], args["mask"],
                           args["o"], args["lse"], args["dout"], args["dq"], args["dk"], args["dv"],
                           args["dbias"], args["ws"], args["ws_bytes"], None)


def detail():
    return _lib.load().evoattn_last_error_detail().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(rows=0), INVALID, "sizes"),
    (dict(n=-1), INVALID, "sizes"),
    (dict(heads=0), INVALID, "sizes"),
    (dict(dtype=7), INVALID, "dtype"),
    (dict(transpose=2), INVALID, "transpose"),
    (dict(head_dim=24), UNSUPPORTED, "head_dim"),
    (dict(head_dim=128), UNSUPPORTED, "head_dim"),
    (dict(rows=1 << 20, n=1 << 10, heads=8, head_dim=64), UNSUPPORTED, "too large"),
    (dict(q=None), INVALID, "q must not be NULL"),
    (dict(v=None), INVALID, "v must not be NULL"),
    (dict(o=None), INVALID, "o must not be NULL"),
    (dict(k=A + 2), INVALID, "aligned"),
    (dict(bias=A + 8), INVALID, "aligned"),
    (dict(mask=A + 2), INVALID, "aligned"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(ws_bytes=16), WORKSPACE, "workspace"),
    (dict(ws=A + 64), INVALID, "256-byte"),
])
def test_fwd_validation(kw, code, needle):
    assert fwd(**kw) == code
    assert needle in detail()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(rows=-3), INVALID, "sizes"),
    (dict(head_dim=12), UNSUPPORTED, "head_dim"),
    (dict(lse=None), INVALID, "lse must not be NULL"),
    (dict(dout=None), INVALID, "dout must not be NULL"),
    (dict(dq=None), INVALID, "dq must not be NULL"),
    (dict(dk=None), INVALID, "dk must not be NULL"),
    (dict(dv=None), INVALID, "dv must not be NULL"),
    (dict(dbias=A + 1), INVALID, "aligned"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(ws_bytes=16), WORKSPACE, "workspace"),
    (dict(ws=A + 64), INVALID, "256-byte"),
])
def test_bwd_validation(kw, code, needle):
    assert bwd(**kw) == code
    assert needle in detail()


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful where no GPU is present")
def test_valid_call_without_device_reports_device_error():
    """A call that passes validation on a machine without a GPU returns EVOATTN_ERR_DEVICE and
    launches nothing (the addresses are fake)."""
    assert fwd() == DEVICE
    assert "device" in detail().lower()


def test_python_binding_rejects_bad_tensors():
    import af3_attention_amd as ea
    q = torch.zeros(2, 3, 1, 8)
    with pytest.raises(ValueError):
        ea.evoattn_fwd(q, q, q)          # CPU tensors are rejected before any library call


def proj(**kw):
    lib = _lib.load()
    args = dict(a=8, b=8, c=128, heads=4, head_dim=32, dtype=1, bt=0, eps=1e-5, x=A, gamma=A, beta=A,
                w_qkv=A, w_bias=A, q=A, k=A, v=A, bias=A, mean=A, rstd=A)
    args.update(kw)
    return lib.evoattn_ln_proj_fwd(args["a"], args["b"], args["c"], args["heads"], args["head_dim"], args["dtype"],
                                   args["bt"], args["eps"], args["x"], args["gamma"], args["beta"], args["w_qkv"],
                                   args["w_bias"], args["q"], args["k"], args["v"], args["bias"], args["mean"],
                                   args["rstd"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(a=0), INVALID, "sizes"),
    (dict(c=-1), INVALID, "sizes"),
    (dict(dtype=3), INVALID, "dtype"),
    (dict(bt=2), INVALID, "bias_transpose"),
    (dict(eps=-1.0), INVALID, "eps"),
    (dict(eps=float("nan")), INVALID, "eps"),
    (dict(w_qkv=None, w_bias=None, q=None, k=None, v=None, bias=None), INVALID, "nothing to project"),
    (dict(head_dim=24), UNSUPPORTED, "head_dim"),
    (dict(c=12), UNSUPPORTED, "channels"),
    (dict(c=4096), UNSUPPORTED, "channels"),
    (dict(c=100), UNSUPPORTED, "channels"),
    (dict(a=8, b=9), INVALID, "square"),
    (dict(a=1 << 16, b=1 << 16, w_bias=None, bias=None), UNSUPPORTED, "too large"),
    (dict(x=None), INVALID, "x must not be NULL"),
    (dict(gamma=None), INVALID, "gamma must not be NULL"),
    (dict(beta=A + 2), INVALID, "aligned"),
    (dict(q=None), INVALID, "q must not be NULL"),
    (dict(v=A + 8), INVALID, "aligned"),
    (dict(w_qkv=None), INVALID, "must be NULL when w_qkv is NULL"),
    (dict(bias=None), INVALID, "bias must not be NULL"),
    (dict(w_bias=None), INVALID, "bias must be NULL"),
    (dict(mean=None), INVALID, "both"),
    (dict(rstd=A + 2), INVALID, "aligned"),
])
def test_ln_proj_fwd_validation(kw, code, needle):
    assert proj(**kw) == code
    assert needle in detail()


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful where no GPU is present")
def test_ln_proj_valid_call_without_device_reports_device_error():
    assert proj() == DEVICE
    assert proj(w_qkv=None, q=None, k=None, v=None, a=5, b=5, mean=None, rstd=None) == DEVICE
    assert proj(w_bias=None, bias=None, a=7, b=3) == DEVICE


def test_ln_proj_binding_rejects_bad_tensors():
    import af3_attention_amd as ea
    x = torch.zeros(2, 2, 16)
    with pytest.raises(ValueError):
        ea.ln_proj_fwd(x, torch.ones(16), torch.zeros(16), heads=1, head_dim=8)


def proj_bwd(**kw):
    lib = _lib.load()
    args = dict(a=8, b=8, c=128, heads=4, head_dim=32, dtype=1, bt=0, x=A, gamma=A, beta=A, w_qkv=A, w_bias=A,
                mean=A, rstd=A, dq=A, dk=A, dv=A, dbias=A, dx=A, dgamma=A, dbeta=A, dw_qkv=A, dw_bias=A, ws=A,
                ws_bytes=1 << 30)
    args.update(kw)
    return lib.evoattn_ln_proj_bwd(*(args[k] for k in (
        "a", "b", "c", "heads", "head_dim", "dtype", "bt", "x", "gamma", "beta", "w_qkv", "w_bias", "mean", "rstd",
        "dq", "dk", "dv", "dbias", "dx", "dgamma", "dbeta", "dw_qkv", "dw_bias", "ws", "ws_bytes")), None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(b=-1), INVALID, "sizes"),
    (dict(head_dim=12), UNSUPPORTED, "head_dim"),
    (dict(a=8, b=7), INVALID, "square"),
    (dict(mean=None), INVALID, "mean must not be NULL"),
    (dict(rstd=None), INVALID, "rstd must not be NULL"),
    (dict(dx=None), INVALID, "dx must not be NULL"),
    (dict(dgamma=None), INVALID, "dgamma must not be NULL"),
    (dict(dbeta=A + 1), INVALID, "aligned"),
    (dict(dq=None), INVALID, "dq must not be NULL"),
    (dict(dw_qkv=None), INVALID, "dw_qkv must not be NULL"),
    (dict(dbias=None), INVALID, "dbias must not be NULL"),
    (dict(dw_bias=None), INVALID, "dw_bias must not be NULL"),
    (dict(w_qkv=None), INVALID, "must be NULL when w_qkv is NULL"),
    (dict(w_bias=None), INVALID, "must be NULL when w_bias is NULL"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(ws_bytes=16), WORKSPACE, "workspace"),
    (dict(ws=A + 64), INVALID, "256-byte"),
])
def test_ln_proj_bwd_validation(kw, code, needle):
    assert proj_bwd(**kw) == code
    assert needle in detail()


def test_ln_proj_bwd_workspace_query():
    lib = _lib.load()
    fixed = 64 * 416 * 128 * 4 + 64 * 416 * 4 + 2 * 388 * 128 * 4 + 5 * 256
    for n_tok in (384, 1536):
        n = lib.evoattn_ln_proj_bwd_workspace_bytes(n_tok, n_tok, 128, 4, 32, 1, 1, 1)
        assert n % 256 == 0
        # partial sums over at most 64 token ranges of a (3*H*d + H, padded to 32) x C array, two
        # (3*H*d + H) x C product arrays, and the pair-bias gradient in token order (16 bf16 per token)
        assert n_tok * n_tok * 16 * 2 <= n <= fixed + n_tok * n_tok * 16 * 2
    # without the bias there is no token-order buffer
    assert lib.evoattn_ln_proj_bwd_workspace_bytes(1536, 1536, 128, 4, 32, 1, 1, 0) <= fixed
    assert lib.evoattn_ln_proj_bwd_workspace_bytes(8, 9, 128, 4, 32, 1, 1, 1) == 0   # bias needs a == b
    assert lib.evoattn_ln_proj_bwd_workspace_bytes(8, 8, 128, 4, 32, 1, 0, 0) == 0   # nothing to project


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful where no GPU is present")
def test_ln_proj_bwd_valid_call_without_device_reports_device_error():
    assert proj_bwd() == DEVICE


def trans_fwd(**kw):
    lib = _lib.load()
    args = dict(a=8, b=8, c=128, n=4, dtype=1, eps=1e-5, x=A, gamma=A, beta=A, wa=A, wb=A, wo=A, out=A, mean=A, rstd=A)
    args.update(kw)
    return lib.evoattn_transition_fwd(*(args[k] for k in ("a", "b", "c", "n", "dtype", "eps", "x", "gamma", "beta",
                                                          "wa", "wb", "wo", "out", "mean", "rstd")), None)


def trans_bwd(**kw):
    lib = _lib.load()
    args = dict(a=8, b=8, c=64, n=4, dtype=1, x=A, gamma=A, beta=A, wa=A, wb=A, wo=A, mean=A, rstd=A, dout=A, dx=A,
                dgamma=A, dbeta=A, dwa=A, dwb=A, dwo=A, ws=A, ws_bytes=1 << 30)
    args.update(kw)
    return lib.evoattn_transition_bwd(*(args[k] for k in (
        "a", "b", "c", "n", "dtype", "x", "gamma", "beta", "wa", "wb", "wo", "mean", "rstd", "dout", "dx", "dgamma",
        "dbeta", "dwa", "dwb", "dwo", "ws", "ws_bytes")), None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(a=0), INVALID, "sizes"),
    (dict(n=0), INVALID, "sizes"),
    (dict(dtype=5), INVALID, "dtype"),
    (dict(eps=-1.0), INVALID, "eps"),
    (dict(dtype=0), UNSUPPORTED, "bf16"),
    (dict(c=96), UNSUPPORTED, "channels"),
    (dict(n=17), UNSUPPORTED, "expansion"),
    (dict(a=1 << 14, b=1 << 14), UNSUPPORTED, "too large"),
    (dict(x=None), INVALID, "x must not be NULL"),
    (dict(wo=None), INVALID, "w_out must not be NULL"),
    (dict(wa=A + 4), INVALID, "aligned"),
    (dict(out=None), INVALID, "out must not be NULL"),
    (dict(mean=None), INVALID, "both"),
])
def test_transition_fwd_validation(kw, code, needle):
    assert trans_fwd(**kw) == code
    assert needle in detail()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(c=32), UNSUPPORTED, "channels"),
    (dict(mean=None), INVALID, "mean must not be NULL"),
    (dict(dout=None), INVALID, "dout must not be NULL"),
    (dict(dx=A + 2), INVALID, "aligned"),
    (dict(dwo=None), INVALID, "dw_out must not be NULL"),
    (dict(ws=None), WORKSPACE, "workspace"),
    (dict(ws_bytes=64), WORKSPACE, "workspace"),
    (dict(ws=A + 64), INVALID, "256-byte"),
])
def test_transition_bwd_validation(kw, code, needle):
    assert trans_bwd(**kw) == code
    assert needle in detail()


def test_transition_workspace_query():
    lib = _lib.load()
    n = lib.evoattn_transition_bwd_workspace_bytes(384, 384, 128, 4, 1)
    assert n % 256 == 0
    # partial sums over at most 64 ranges of three n*C x C arrays, two n*C vectors, two n*C x C products,
    # and the normalised input rows in bf16
    hc = 512 * 128 * 4
    xh = 384 * 384 * 128 * 2
    assert n >= xh
    assert n <= 64 * (3 * hc + 2 * 512 * 4) + 2 * hc + xh + 9 * 256
    assert lib.evoattn_transition_bwd_workspace_bytes(384, 384, 128, 4, 0) == 0   # fp32: unsupported


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful where no GPU is present")
def test_transition_valid_call_without_device_reports_device_error():
    assert trans_fwd() == DEVICE
    assert trans_bwd() == DEVICE
