"""MI355X-native memory-efficient 3D attention with an additively broadcast pair bias.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
declared in include/evoattn.h; this package is the thin Python binding.
"""
from .evoattn import (  # noqa: F401
    EvoAttnFunction,
    evoattn,
    evoattn_bwd,
    evoattn_bwd_workspace_bytes,
    evoattn_fwd,
    evoattn_fwd_noalloc,
    evoattn_fwd_workspace_bytes,
)
from ._lib import EvoAttnError, LIB_PATH  # noqa: F401
from .evofusion import (  # noqa: F401,E402
    LNProjFunction, TransitionFunction, ln_proj, ln_proj_bwd, ln_proj_bwd_workspace_bytes, ln_proj_fwd, transition,
    transition_bwd, transition_bwd_workspace_bytes, transition_fwd)
