"""Engram gate for AMD MI355X: Python binding of the HIP library libtk_engram.so.

The gate (zhichai.net TileKernels page, section "5. Engram", gate formula):
    d    = <RMSNorm of x with weight wh, RMSNorm of k with weight we>
    gate = sigmoid(sign(d) * sqrt(|d| / sqrt(H)))
    out  = x + gate * v
with its backward (dx, dk, dv) and the weight-gradient reduction (dwh, dwe).
The C ABI is declared in include/tk_engram.h; the functions below have the
same names and only marshal torch tensors into it.
"""

from ._binding import (  # noqa: F401
    DSQRT_CLAMP,
    BoundCall,
    bind_fused_weight,
    bind_gate_bwd,
    bind_gate_fwd,
    bind_grad_w_reduce,
    EPS,
    EXPORTS,
    TkError,
    load_library,
    tk_abi_version,
    tk_engram_bwd_workspace_bytes,
    tk_engram_copy_probe,
    tk_engram_gate_bwd,
    tk_engram_gate_bwd_fused,
    tk_engram_gate_bwd_reduce_noalloc,
    tk_engram_gate_fwd,
    tk_engram_gate_fwd_fused,
    tk_engram_gate_launches,
    tk_engram_grad_w_reduce,
    tk_engram_fused_weight,
    tk_engram_gather,
    tk_engram_hash,
    tk_engram_num_partials,
    tk_engram_stream_probe,
    tk_status_string,
)
from .build import LIB as LIBRARY_PATH  # noqa: F401

# The autograd wrapper imports torch; load it on first use.
_AUTOGRAD = ("EngramGateFunction", "EngramGate", "engram_gate")


def __getattr__(name):
    if name in _AUTOGRAD:
        from . import autograd
        return getattr(autograd, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")

