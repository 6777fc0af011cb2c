"""ctypes binding of libtk_engram.so (declared in include/tk_engram.h).

Argument marshalling only: tensors are checked for dtype, shape, device and
contiguity, their device pointers and the current HIP stream are passed to
the C ABI, and a nonzero status raises.  Every step of the gate runs in the
library's HIP kernels; there is no other implementation to fall back to, and
a missing library raises.
"""

from __future__ import annotations

import ctypes
import os

from .build import LIB

EPS = 1e-6            # RMSNorm epsilon
DSQRT_CLAMP = 1e-4    # lower clamp of |z| in the signed-sqrt derivative

TK_SUCCESS = 0
TK_ERR_NULL = 1
TK_ERR_SHAPE = 2
TK_ERR_ALIGN = 3
TK_ERR_UNSUPPORTED = 4
TK_ERR_WORKSPACE = 5
TK_ERR_LAUNCH = 6
TK_ERR_VALUE = 7

EXPORTS = (
    "tk_engram_gate_fwd", "tk_engram_gate_bwd", "tk_engram_grad_w_reduce",
    "tk_engram_num_partials", "tk_engram_bwd_workspace_bytes",
    "tk_engram_copy_probe", "tk_status_string", "tk_abi_version", "tk_engram_hash",
    "tk_engram_gather", "tk_engram_fused_weight", "tk_engram_stream_probe",
    "tk_engram_gate_bwd_reduce_noalloc", "tk_engram_gate_fwd_fused",
    "tk_engram_gate_bwd_fused", "tk_engram_gate_launches",
)

HASH_MAX_NGRAM = 4


class TkError(RuntimeError):
    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call}: {message} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB) -> ctypes.CDLL:
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with __graft_entry__.build() "
            "(the Engram gate has no implementation other than its HIP kernels)")
    L = ctypes.CDLL(path)
    vp, i64, sz, dbl, i32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_double, ctypes.c_int32)
    L.tk_engram_gate_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, dbl, vp]
    L.tk_engram_gate_fwd.restype = i32
    L.tk_engram_gate_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                     i64, i64, dbl, dbl, vp]
    L.tk_engram_gate_bwd.restype = i32
    L.tk_engram_grad_w_reduce.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    L.tk_engram_grad_w_reduce.restype = i32
    L.tk_engram_gate_fwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, dbl, vp]
    L.tk_engram_gate_fwd_fused.restype = i32
    L.tk_engram_gate_bwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                           i64, i64, dbl, dbl, vp]
    L.tk_engram_gate_bwd_fused.restype = i32
    L.tk_engram_gate_bwd_reduce_noalloc.argtypes = [vp] * 11 + [i64, i64, dbl, dbl, vp]
    L.tk_engram_gate_bwd_reduce_noalloc.restype = i32
    L.tk_engram_num_partials.argtypes = [i64, i64]
    L.tk_engram_num_partials.restype = i64
    L.tk_engram_gate_launches.argtypes = [i64, i64, i32]
    L.tk_engram_gate_launches.restype = i64
    L.tk_engram_bwd_workspace_bytes.argtypes = [i64, i64]
    L.tk_engram_bwd_workspace_bytes.restype = sz
    L.tk_engram_copy_probe.argtypes = [vp, vp, sz, vp]
    L.tk_engram_copy_probe.restype = i32
    L.tk_status_string.argtypes = [i32]
    L.tk_status_string.restype = ctypes.c_char_p
    L.tk_abi_version.argtypes = []
    L.tk_abi_version.restype = i32
    L.tk_engram_hash.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, ctypes.c_uint32, vp, vp]
    L.tk_engram_hash.restype = i32
    L.tk_engram_gather.argtypes = [vp, i64, i32, vp, i64, i64, vp, vp, vp, vp]
    L.tk_engram_gather.restype = i32
    L.tk_engram_fused_weight.argtypes = [vp, vp, vp, i64, vp]
    L.tk_engram_fused_weight.restype = i32
    L.tk_engram_stream_probe.argtypes = [vp, i32, vp, i32, sz, vp]
    L.tk_engram_stream_probe.restype = i32
    _lib = L
    return L


def tk_status_string(status: int) -> str:
    return load_library().tk_status_string(status).decode()


def tk_abi_version() -> int:
    return int(load_library().tk_abi_version())


def tk_engram_num_partials(T: int, H: int) -> int:
    return int(load_library().tk_engram_num_partials(T, H))


def tk_engram_gate_launches(T: int, H: int, backward: bool) -> int:
    return int(load_library().tk_engram_gate_launches(T, H, 1 if backward else 0))


def tk_engram_bwd_workspace_bytes(T: int, H: int) -> int:
    return int(load_library().tk_engram_bwd_workspace_bytes(T, H))


def _check(call: str, status: int) -> None:
    if status != TK_SUCCESS:
        raise TkError(call, status, tk_status_string(status))


# ---- tensor marshalling ----------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _rows(x, name="x"):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D [T, H] tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    return x.shape[0], x.shape[1], x.device


def tk_engram_gate_fwd(x, k, v, wh, we, out=None, gate=None, eps=EPS, stream=None):
    """out = x + gate * v and gate [T] (fp32); x, k, v bf16 [T, H]."""
    torch = _torch()
    T, H, dev = _rows(x)
    bf, f32 = torch.bfloat16, torch.float32
    if out is None:
        out = torch.empty((T, H), dtype=bf, device=dev)
    if gate is None:
        gate = torch.empty((T,), dtype=f32, device=dev)
    args = [_need(x, "x", bf, (T, H), dev), _need(k, "k", bf, (T, H), dev),
            _need(v, "v", bf, (T, H), dev), _need(wh, "wh", f32, (H,), dev),
            _need(we, "we", f32, (H,), dev), _need(out, "out", bf, (T, H), dev),
            _need(gate, "gate", f32, (T,), dev)]
    st = load_library().tk_engram_gate_fwd(*args, T, H, float(eps),
                                           _stream_handle(dev, stream))
    _check("tk_engram_gate_fwd", st)
    return out, gate


def tk_engram_gate_bwd(grad_out, x, k, v, wh, we, dx=None, dk=None, dv=None,
                       workspace=None, eps=EPS, dsqrt_clamp=DSQRT_CLAMP, stream=None):
    """dx, dk, dv (bf16 [T, H]) and the fp32 [P, H] weight-gradient partials."""
    torch = _torch()
    T, H, dev = _rows(x)
    bf, f32 = torch.bfloat16, torch.float32
    P = tk_engram_num_partials(T, H)
    if dx is None:
        dx = torch.empty((T, H), dtype=bf, device=dev)
    if dk is None:
        dk = torch.empty((T, H), dtype=bf, device=dev)
    if dv is None:
        dv = torch.empty((T, H), dtype=bf, device=dev)
    if workspace is None:
        workspace = torch.empty((max(P, 1), H), dtype=f32, device=dev)
    if workspace.dtype != f32 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous fp32 GPU tensor")
    args = [_need(grad_out, "grad_out", bf, (T, H), dev), _need(x, "x", bf, (T, H), dev),
            _need(k, "k", bf, (T, H), dev), _need(v, "v", bf, (T, H), dev),
            _need(wh, "wh", f32, (H,), dev), _need(we, "we", f32, (H,), dev),
            _need(dx, "dx", bf, (T, H), dev), _need(dk, "dk", bf, (T, H), dev),
            _need(dv, "dv", bf, (T, H), dev), ctypes.c_void_p(workspace.data_ptr())]
    st = load_library().tk_engram_gate_bwd(*args, workspace.numel() * 4, T, H,
                                           float(eps), float(dsqrt_clamp),
                                           _stream_handle(dev, stream))
    _check("tk_engram_gate_bwd", st)
    return dx, dk, dv, workspace, P


def tk_engram_gate_fwd_fused(x, k, v, w, out=None, gate=None, eps=EPS, stream=None):
    """tk_engram_gate_fwd with the fused weight w = wh * we (fp64 [H])."""
    torch = _torch()
    T, H, dev = _rows(x)
    bf, f32 = torch.bfloat16, torch.float32
    out = torch.empty((T, H), dtype=bf, device=dev) if out is None else out
    gate = torch.empty((T,), dtype=f32, device=dev) if gate is None else gate
    args = [_need(x, "x", bf, (T, H), dev), _need(k, "k", bf, (T, H), dev),
            _need(v, "v", bf, (T, H), dev), _need(w, "w", torch.float64, (H,), dev),
            _need(out, "out", bf, (T, H), dev), _need(gate, "gate", f32, (T,), dev)]
    st = load_library().tk_engram_gate_fwd_fused(*args, T, H, float(eps),
                                                 _stream_handle(dev, stream))
    _check("tk_engram_gate_fwd_fused", st)
    return out, gate


def tk_engram_gate_bwd_fused(grad_out, x, k, v, w, dx=None, dk=None, dv=None, workspace=None,
                             eps=EPS, dsqrt_clamp=DSQRT_CLAMP, stream=None):
    """tk_engram_gate_bwd with the fused weight w = wh * we (fp64 [H])."""
    torch = _torch()
    T, H, dev = _rows(x)
    bf, f32 = torch.bfloat16, torch.float32
    P = tk_engram_num_partials(T, H)
    dx = torch.empty((T, H), dtype=bf, device=dev) if dx is None else dx
    dk = torch.empty((T, H), dtype=bf, device=dev) if dk is None else dk
    dv = torch.empty((T, H), dtype=bf, device=dev) if dv is None else dv
    if workspace is None:
        workspace = torch.empty((max(P, 1), H), dtype=f32, device=dev)
    if workspace.dtype != f32 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous fp32 GPU tensor")
    args = [_need(grad_out, "grad_out", bf, (T, H), dev), _need(x, "x", bf, (T, H), dev),
            _need(k, "k", bf, (T, H), dev), _need(v, "v", bf, (T, H), dev),
            _need(w, "w", torch.float64, (H,), dev), _need(dx, "dx", bf, (T, H), dev),
            _need(dk, "dk", bf, (T, H), dev), _need(dv, "dv", bf, (T, H), dev),
            ctypes.c_void_p(workspace.data_ptr())]
    st = load_library().tk_engram_gate_bwd_fused(*args, workspace.numel() * 4, T, H,
                                                 float(eps), float(dsqrt_clamp),
                                                 _stream_handle(dev, stream))
    _check("tk_engram_gate_bwd_fused", st)
    return dx, dk, dv, workspace, P


def tk_engram_grad_w_reduce(workspace, P, H, wh, we, dwh=None, dwe=None, stream=None):
    """dwh = we * sum_p workspace[p], dwe = wh * sum_p workspace[p] (fp32 [H])."""
    torch = _torch()
    dev = wh.device
    f32 = torch.float32
    if workspace.dtype != f32 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous fp32 tensor on wh's device")
    if workspace.numel() < P * H:
        raise ValueError("workspace holds fewer than P * H values")
    if dwh is None:
        dwh = torch.empty((H,), dtype=f32, device=dev)
    if dwe is None:
        dwe = torch.empty((H,), dtype=f32, device=dev)
    st = load_library().tk_engram_grad_w_reduce(
        ctypes.c_void_p(workspace.data_ptr()), P, H, _need(wh, "wh", f32, (H,), dev),
        _need(we, "we", f32, (H,), dev), _need(dwh, "dwh", f32, (H,), dev),
        _need(dwe, "dwe", f32, (H,), dev), _stream_handle(dev, stream))
    _check("tk_engram_grad_w_reduce", st)
    return dwh, dwe


def tk_engram_gate_bwd_reduce_noalloc(grad_out, x, k, v, wh, we, dx=None, dk=None, dv=None,
                                      dwh=None, dwe=None, eps=EPS, dsqrt_clamp=DSQRT_CLAMP,
                                      stream=None):
    """dx, dk, dv (bf16 [T, H]) and dwh, dwe (fp32 [H]) in one call whose
    weight-gradient partials stay in the library's own device memory; the
    C call allocates nothing (outputs left as None are allocated here)."""
    torch = _torch()
    T, H, dev = _rows(x)
    bf, f32 = torch.bfloat16, torch.float32
    dx = torch.empty((T, H), dtype=bf, device=dev) if dx is None else dx
    dk = torch.empty((T, H), dtype=bf, device=dev) if dk is None else dk
    dv = torch.empty((T, H), dtype=bf, device=dev) if dv is None else dv
    dwh = torch.empty((H,), dtype=f32, device=dev) if dwh is None else dwh
    dwe = torch.empty((H,), dtype=f32, device=dev) if dwe is None else dwe
    args = [_need(grad_out, "grad_out", bf, (T, H), dev), _need(x, "x", bf, (T, H), dev),
            _need(k, "k", bf, (T, H), dev), _need(v, "v", bf, (T, H), dev),
            _need(wh, "wh", f32, (H,), dev), _need(we, "we", f32, (H,), dev),
            _need(dx, "dx", bf, (T, H), dev), _need(dk, "dk", bf, (T, H), dev),
            _need(dv, "dv", bf, (T, H), dev), _need(dwh, "dwh", f32, (H,), dev),
            _need(dwe, "dwe", f32, (H,), dev)]
    st = load_library().tk_engram_gate_bwd_reduce_noalloc(
        *args, T, H, float(eps), float(dsqrt_clamp), _stream_handle(dev, stream))
    _check("tk_engram_gate_bwd_reduce_noalloc", st)
    return dx, dk, dv, dwh, dwe


def _probe_tensors(tensors):
    """The probes' tensors: contiguous, on one GPU, of one byte size."""
    torch = _torch()
    dev = tensors[0].device if isinstance(tensors[0], torch.Tensor) else None
    if dev is None or dev.type != "cuda":
        raise ValueError("probe tensors must be GPU tensors")
    n = tensors[0].numel() * tensors[0].element_size()
    for t in tensors:
        if not isinstance(t, torch.Tensor) or t.device != dev:
            raise ValueError(f"all probe tensors must be on {dev}")
        if not t.is_contiguous() or t.numel() * t.element_size() != n:
            raise ValueError("all probe tensors must be contiguous and of one byte size")
    return dev, n


def tk_engram_copy_probe(src, dst, stream=None):
    """Copy src into dst (same byte size) with the library's 128-bit copy."""
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("src and dst differ in size")
    _, n = _probe_tensors([src, dst])
    st = load_library().tk_engram_copy_probe(ctypes.c_void_p(src.data_ptr()),
                                             ctypes.c_void_p(dst.data_ptr()), n,
                                             _stream_handle(src.device, stream))
    _check("tk_engram_copy_probe", st)
    return dst


# ---- pre-marshalled calls ---------------------------------------------------

class BoundCall:
    """One C-ABI call whose arguments were checked and marshalled once.

    Calling it only enqueues the kernels (no tensor checks, no pointer
    lookups), so a timing loop is never limited by Python overhead. It keeps
    references to its tensors, which therefore stay allocated while it lives.
    """

    def __init__(self, name, fn, args, keep):
        self._name, self._fn, self._args, self._keep = name, fn, tuple(args), keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != TK_SUCCESS:
            _check(self._name, st)


def bind_gate_fwd(x, k, v, wh, we, out, gate, eps=EPS, stream=None):
    """tk_engram_gate_fwd with fixed arguments; see tk_engram_gate_fwd."""
    torch = _torch()
    T, H, dev = _rows(x)
    bf, f32 = torch.bfloat16, torch.float32
    args = [_need(x, "x", bf, (T, H), dev), _need(k, "k", bf, (T, H), dev),
            _need(v, "v", bf, (T, H), dev), _need(wh, "wh", f32, (H,), dev),
            _need(we, "we", f32, (H,), dev), _need(out, "out", bf, (T, H), dev),
            _need(gate, "gate", f32, (T,), dev), ctypes.c_int64(T), ctypes.c_int64(H),
            ctypes.c_double(eps), _stream_handle(dev, stream)]
    return BoundCall("tk_engram_gate_fwd", load_library().tk_engram_gate_fwd, args,
                     (x, k, v, wh, we, out, gate))


def bind_gate_bwd(grad_out, x, k, v, wh, we, dx, dk, dv, workspace, eps=EPS,
                  dsqrt_clamp=DSQRT_CLAMP, stream=None):
    """tk_engram_gate_bwd with fixed arguments; see tk_engram_gate_bwd."""
    torch = _torch()
    T, H, dev = _rows(x)
    bf, f32 = torch.bfloat16, torch.float32
    if workspace.dtype != f32 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous fp32 GPU tensor")
    args = [_need(grad_out, "grad_out", bf, (T, H), dev), _need(x, "x", bf, (T, H), dev),
            _need(k, "k", bf, (T, H), dev), _need(v, "v", bf, (T, H), dev),
            _need(wh, "wh", f32, (H,), dev), _need(we, "we", f32, (H,), dev),
            _need(dx, "dx", bf, (T, H), dev), _need(dk, "dk", bf, (T, H), dev),
            _need(dv, "dv", bf, (T, H), dev), ctypes.c_void_p(workspace.data_ptr()),
            ctypes.c_size_t(workspace.numel() * 4), ctypes.c_int64(T), ctypes.c_int64(H),
            ctypes.c_double(eps), ctypes.c_double(dsqrt_clamp), _stream_handle(dev, stream)]
    return BoundCall("tk_engram_gate_bwd", load_library().tk_engram_gate_bwd, args,
                     (grad_out, x, k, v, wh, we, dx, dk, dv, workspace))


def bind_grad_w_reduce(workspace, P, H, wh, we, dwh, dwe, stream=None):
    """tk_engram_grad_w_reduce with fixed arguments; see tk_engram_grad_w_reduce."""
    torch = _torch()
    dev = wh.device
    f32 = torch.float32
    if workspace.dtype != f32 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous fp32 tensor on wh's device")
    if workspace.numel() < P * H:
        raise ValueError("workspace holds fewer than P * H values")
    args = [ctypes.c_void_p(workspace.data_ptr()), ctypes.c_int64(P), ctypes.c_int64(H),
            _need(wh, "wh", f32, (H,), dev), _need(we, "we", f32, (H,), dev),
            _need(dwh, "dwh", f32, (H,), dev), _need(dwe, "dwe", f32, (H,), dev),
            _stream_handle(dev, stream)]
    return BoundCall("tk_engram_grad_w_reduce", load_library().tk_engram_grad_w_reduce,
                     args, (workspace, wh, we, dwh, dwe))


# ---- N-gram hash --------------------------------------------------------------

def _host_array(a, dtype, shape, name):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=dtype)
    if a.shape != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {a.shape}")
    return a


def tk_engram_hash(tokens, ngram, mult, table_size, pad, out=None, stream=None):
    """Table indices int32 [B, S, L, K] of the N-gram hash of `tokens` (int32
    [B, S] on the GPU). ngram [L], mult uint64 [L, K, 4] and table_size uint32
    [L, K] are host arrays (numpy or lists)."""
    import numpy as np
    torch = _torch()
    if not isinstance(tokens, torch.Tensor) or tokens.dim() != 2:
        raise ValueError("tokens must be a 2-D [B, S] tensor")
    if tokens.device.type != "cuda":
        raise ValueError("tokens must be a GPU tensor")
    B, S = tokens.shape
    dev = tokens.device
    table_size = np.ascontiguousarray(table_size, dtype=np.uint32)
    if table_size.ndim != 2:
        raise ValueError("table_size must be [L, K]")
    L, K = table_size.shape
    ngram = _host_array(ngram, np.int32, (L,), "ngram")
    mult = _host_array(mult, np.uint64, (L, K, HASH_MAX_NGRAM), "mult")
    if out is None:
        out = torch.empty((B, S, L, K), dtype=torch.int32, device=dev)
    tp = _need(tokens, "tokens", torch.int32, (B, S), dev)
    op = _need(out, "out", torch.int32, (B, S, L, K), dev)
    st = load_library().tk_engram_hash(
        tp, B, S, L, K, ctypes.c_void_p(ngram.ctypes.data), ctypes.c_void_p(mult.ctypes.data),
        ctypes.c_void_p(table_size.ctypes.data), int(pad) & 0xFFFFFFFF, op,
        _stream_handle(dev, stream))
    _check("tk_engram_hash", st)
    return out


# ---- hashed multi-table gather ---------------------------------------------------

def tk_engram_gather(idx, table_data, row_offset, rows, out=None, stream=None):
    """out [T, Q, d] bf16: row row_offset[q] + idx[t, q] of `table_data` (bf16
    [R, d] on the GPU) for every token t and table q; a zero row where the
    index is outside table q. idx is int32 [T, Q] (or [..., Q], flattened) on
    the GPU; row_offset (int64) and rows (uint32) are host arrays of length Q."""
    import numpy as np
    torch = _torch()
    if not isinstance(idx, torch.Tensor) or idx.dim() < 1 or idx.device.type != "cuda":
        raise ValueError("idx must be an int32 GPU tensor [..., Q]")
    if not isinstance(table_data, torch.Tensor) or table_data.dim() != 2:
        raise ValueError("table_data must be a 2-D [R, d] tensor")
    Q = idx.shape[-1]
    lead = tuple(idx.shape[:-1])
    T = int(np.prod(lead)) if lead else 1
    R, d = table_data.shape
    dev = idx.device
    row_offset = _host_array(row_offset, np.int64, (Q,), "row_offset")
    rows = _host_array(rows, np.uint32, (Q,), "rows")
    if not idx.is_contiguous():
        # no hidden copy: a temporary freed on return could still be in use
        # by the kernel on a side stream
        raise ValueError("idx must be contiguous")
    idx2 = idx.view(T, Q)
    if out is None:
        out = torch.empty((*lead, Q, d), dtype=torch.bfloat16, device=dev)
    ip = _need(idx2, "idx", torch.int32, (T, Q), dev)
    tp = _need(table_data, "table_data", torch.bfloat16, (R, d), dev)
    op = _need(out.view(T, Q, d), "out", torch.bfloat16, (T, Q, d), dev)
    st = load_library().tk_engram_gather(
        ip, T, Q, tp, R, d, ctypes.c_void_p(row_offset.ctypes.data),
        ctypes.c_void_p(rows.ctypes.data), op, _stream_handle(dev, stream))
    _check("tk_engram_gather", st)
    return out


def bind_fused_weight(wh, we, w, stream=None):
    """tk_engram_fused_weight with fixed arguments; see tk_engram_fused_weight."""
    torch = _torch()
    if not isinstance(wh, torch.Tensor) or wh.dim() != 1 or wh.device.type != "cuda":
        raise ValueError("wh must be a 1-D fp32 GPU tensor")
    H = wh.shape[0]
    dev = wh.device
    args = [_need(wh, "wh", torch.float32, (H,), dev), _need(we, "we", torch.float32, (H,), dev),
            _need(w, "w", torch.float64, (H,), dev), ctypes.c_int64(H),
            _stream_handle(dev, stream)]
    return BoundCall("tk_engram_fused_weight", load_library().tk_engram_fused_weight, args,
                     (wh, we, w))


def tk_engram_fused_weight(wh, we, w=None, stream=None):
    """w = wh * we in fp64 (exact), from fp32 [H] GPU tensors."""
    torch = _torch()
    if not isinstance(wh, torch.Tensor) or wh.dim() != 1 or wh.device.type != "cuda":
        raise ValueError("wh must be a 1-D fp32 GPU tensor")
    H = wh.shape[0]
    dev = wh.device
    if w is None:
        w = torch.empty((H,), dtype=torch.float64, device=dev)
    st = load_library().tk_engram_fused_weight(
        _need(wh, "wh", torch.float32, (H,), dev), _need(we, "we", torch.float32, (H,), dev),
        _need(w, "w", torch.float64, (H,), dev), H, _stream_handle(dev, stream))
    _check("tk_engram_fused_weight", st)
    return w


def tk_engram_stream_probe(srcs, dsts, stream=None):
    """Stream every tensor of `srcs` in and write every tensor of `dsts` (all
    GPU tensors of one byte size) with the library's tiled probe kernel."""
    if not srcs or not dsts:
        raise ValueError("need at least one source and one destination")
    _, n = _probe_tensors(list(srcs) + list(dsts))
    src = (ctypes.c_void_p * len(srcs))(*[t.data_ptr() for t in srcs])
    dst = (ctypes.c_void_p * len(dsts))(*[t.data_ptr() for t in dsts])
    st = load_library().tk_engram_stream_probe(
        ctypes.cast(src, ctypes.c_void_p), len(srcs), ctypes.cast(dst, ctypes.c_void_p),
        len(dsts), n, _stream_handle(srcs[0].device, stream))
    _check("tk_engram_stream_probe", st)

