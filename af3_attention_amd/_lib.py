"""ctypes loader for libevoattn.so.  Loading fails loudly if the library is not built."""
from __future__ import annotations

import ctypes
import os

# EVOATTN_LIB names another build of the library (the sanitizer build of the CPU
# ABI tests); by default the one built in the package directory.
LIB_PATH = os.environ.get("EVOATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libevoattn.so")

EXPORTS = (
    "evoattn_abi_version",
    "evoattn_status_string",
    "evoattn_last_error_detail",
    "evoattn_fwd_workspace_bytes",
    "evoattn_bwd_workspace_bytes",
    "evoattn_fwd",
    "evoattn_fwd_noalloc",
    "evoattn_bwd",
    "evoattn_timing_enable",
    "evoattn_timing_collect",
    "evoattn_ln_proj_fwd",
    "evoattn_ln_proj_bwd_workspace_bytes",
    "evoattn_ln_proj_bwd",
    "evoattn_transition_fwd",
    "evoattn_transition_bwd_workspace_bytes",
    "evoattn_transition_bwd",
)

_lib = None


def load():
    """Returns the loaded library with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m af3_attention_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, c_int, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    fp = ctypes.c_void_p  # float* passed as raw device address
    lib.evoattn_abi_version.argtypes = []
    lib.evoattn_abi_version.restype = c_int
    lib.evoattn_status_string.argtypes = [c_int]
    lib.evoattn_status_string.restype = ctypes.c_char_p
    lib.evoattn_last_error_detail.argtypes = []
    lib.evoattn_last_error_detail.restype = ctypes.c_char_p
    for name in ("evoattn_fwd_workspace_bytes", "evoattn_bwd_workspace_bytes"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, i64, c_int]
        f.restype = sz
    lib.evoattn_fwd.argtypes = [i64, i64, i64, i64, c_int, c_int,
                                vp, vp, vp, vp, fp, vp, fp, vp, sz, vp]
    lib.evoattn_fwd.restype = c_int
    lib.evoattn_fwd_noalloc.argtypes = [i64, i64, i64, i64, c_int, c_int,
                                        vp, vp, vp, vp, fp, vp, fp, vp]
    lib.evoattn_fwd_noalloc.restype = c_int
    lib.evoattn_bwd.argtypes = [i64, i64, i64, i64, c_int, c_int,
                                vp, vp, vp, vp, fp, vp, fp, vp, vp, vp, vp, fp, vp, sz, vp]
    lib.evoattn_bwd.restype = c_int
    lib.evoattn_ln_proj_fwd.argtypes = [i64, i64, i64, i64, i64, c_int, c_int, ctypes.c_float,
                                        vp, fp, fp, vp, vp, vp, vp, vp, vp, fp, fp, vp]
    lib.evoattn_ln_proj_fwd.restype = c_int
    lib.evoattn_ln_proj_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, c_int, c_int, c_int]
    lib.evoattn_ln_proj_bwd_workspace_bytes.restype = sz
    lib.evoattn_ln_proj_bwd.argtypes = [i64, i64, i64, i64, i64, c_int, c_int, vp, fp, fp, vp, vp, fp, fp,
                                        vp, vp, vp, fp, vp, fp, fp, fp, fp, vp, sz, vp]
    lib.evoattn_ln_proj_bwd.restype = c_int
    lib.evoattn_transition_fwd.argtypes = [i64, i64, i64, i64, c_int, ctypes.c_float, vp, fp, fp, vp, vp, vp, vp,
                                           fp, fp, vp]
    lib.evoattn_transition_fwd.restype = c_int
    lib.evoattn_transition_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, c_int]
    lib.evoattn_transition_bwd_workspace_bytes.restype = sz
    lib.evoattn_transition_bwd.argtypes = [i64, i64, i64, i64, c_int, vp, fp, fp, vp, vp, vp, fp, fp, vp, vp, fp, fp,
                                           fp, fp, fp, vp, sz, vp]
    lib.evoattn_transition_bwd.restype = c_int
    lib.evoattn_timing_enable.argtypes = [c_int]
    lib.evoattn_timing_enable.restype = None
    lib.evoattn_timing_collect.argtypes = [c_int, ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_double)]
    lib.evoattn_timing_collect.restype = c_int
    _lib = lib
    return lib


class EvoAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        name = lib.evoattn_status_string(status).decode()
        detail = lib.evoattn_last_error_detail().decode()
        super().__init__(f"{where}: {name}: {detail}")
        self.status = status


def check(status: int, where: str):
    if status != 0:
        raise EvoAttnError(status, where)


def timing_enable(on: bool = True):
    """Bracket every kernel launch of the library with HIP events on its stream."""
    load().evoattn_timing_enable(1 if on else 0)


def timing_collect(max_entries: int = 32):
    """Wait for recorded launches; return {kernel name: (launches, total ms)} and clear the record."""
    lib = load()
    names = ctypes.create_string_buffer(64 * max_entries)
    counts = (ctypes.c_int64 * max_entries)()
    total = (ctypes.c_double * max_entries)()
    n = lib.evoattn_timing_collect(max_entries, names, counts, total)
    if n < 0:
        raise RuntimeError("evoattn_timing_collect: HIP error while reading events")
    out = {}
    for i in range(min(n, max_entries)):
        nm = names.raw[64 * i: 64 * i + 64].split(b"\0", 1)[0].decode()
        out[nm] = (int(counts[i]), float(total[i]))
    return out
