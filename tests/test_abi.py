"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments before any device work."""

import ctypes
import os
import re

import pytest

import engram_conditional_memory_amd as eg
from engram_conditional_memory_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tk_engram.h")

pytestmark = pytest.mark.skipif(not os.path.exists(eg.LIBRARY_PATH),
                                reason="libtk_engram.so not built")

A16 = 0x10000          # a 16-byte-aligned fake device address (never dereferenced)
A4 = 0x10004
B_MAX_PARTIALS = 512   # TK_ENGRAM_MAX_PARTIALS


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tk_\w+)\s*\(", text)))


def test_header_and_library_exports_agree():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    lib = eg.load_library()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert eg.tk_abi_version() == 1
    seen = set()
    for s in range(8):
        msg = eg.tk_status_string(s)
        assert msg and msg not in seen
        seen.add(msg)
    assert eg.tk_status_string(99) == "unknown status"


def test_partials_are_a_function_of_shape():
    assert eg.tk_engram_num_partials(0, 4096) == 0
    assert eg.tk_engram_bwd_workspace_bytes(0, 4096) == 0
    for T, H in ((1, 8), (64, 256), (1024, 4096), (16384, 4096), (32768, 7168),
                 (65537, 7168)):
        P = eg.tk_engram_num_partials(T, H)
        # rows are dealt to P blocks in turn (row t to block t mod P), so
        # every block owns at least one row exactly when P <= T
        assert 1 <= P <= T
        assert P == eg.tk_engram_num_partials(T, H)
        assert eg.tk_engram_bwd_workspace_bytes(T, H) == P * H * 4
    assert eg.tk_engram_num_partials(64, 12) == 0      # invalid shapes give 0
    assert eg.tk_engram_num_partials(-1, 64) == 0


def test_launch_counts_are_a_function_of_shape():
    # the row walk in epochs of about 240 MB of each [T, H] tensor
    assert eg.tk_engram_gate_launches(0, 7168, True) == 0
    assert eg.tk_engram_gate_launches(64, 12, False) == 0
    for backward in (False, True):
        assert eg.tk_engram_gate_launches(1024, 4096, backward) == 1
        assert eg.tk_engram_gate_launches(16384, 4096, backward) == 1
        # H = 7168: 224 blocks, 240 MiB / (224 * 14336 B) = 78 rows per block
        assert eg.tk_engram_gate_launches(224 * 78, 7168, backward) == 1
        assert eg.tk_engram_gate_launches(224 * 78 + 1, 7168, backward) == 2
        assert eg.tk_engram_gate_launches(32768, 7168, backward) == 2
        assert eg.tk_engram_gate_launches(65537, 7168, backward) == 4
        # H = 4096: 256 blocks, 120 rows per block
        assert eg.tk_engram_gate_launches(40000, 4096, backward) == 2


def fwd(**kw):
    a = dict(x=A16, k=A16, v=A16, wh=A16, we=A16, out=A16, gate=A16, T=4, H=64,
             eps=1e-6)
    a.update(kw)
    return eg.load_library().tk_engram_gate_fwd(
        a["x"], a["k"], a["v"], a["wh"], a["we"], a["out"], a["gate"], a["T"], a["H"],
        a["eps"], None)


def bwd(**kw):
    a = dict(g=A16, x=A16, k=A16, v=A16, wh=A16, we=A16, dx=A16, dk=A16, dv=A16,
             ws=A16, wsb=1 << 30, T=4, H=64, eps=1e-6, clamp=1e-4)
    a.update(kw)
    return eg.load_library().tk_engram_gate_bwd(
        a["g"], a["x"], a["k"], a["v"], a["wh"], a["we"], a["dx"], a["dk"], a["dv"],
        a["ws"], a["wsb"], a["T"], a["H"], a["eps"], a["clamp"], None)


def red(**kw):
    a = dict(ws=A16, P=3, H=64, wh=A16, we=A16, dwh=A16, dwe=A16)
    a.update(kw)
    return eg.load_library().tk_engram_grad_w_reduce(
        a["ws"], a["P"], a["H"], a["wh"], a["we"], a["dwh"], a["dwe"], None)


def noalloc(**kw):
    a = dict(g=A16, x=A16, k=A16, v=A16, wh=A16, we=A16, dx=A16, dk=A16, dv=A16,
             dwh=A16, dwe=A16, T=4, H=64, eps=1e-6, clamp=1e-4)
    a.update(kw)
    return eg.load_library().tk_engram_gate_bwd_reduce_noalloc(
        a["g"], a["x"], a["k"], a["v"], a["wh"], a["we"], a["dx"], a["dk"], a["dv"],
        a["dwh"], a["dwe"], a["T"], a["H"], a["eps"], a["clamp"], None)


def test_forward_argument_checks():
    assert fwd(T=-1) == B.TK_ERR_SHAPE
    assert fwd(H=0) == B.TK_ERR_SHAPE
    assert fwd(H=12) == B.TK_ERR_ALIGN
    assert fwd(H=8200) == B.TK_ERR_UNSUPPORTED
    assert fwd(eps=0.0) == B.TK_ERR_VALUE
    assert fwd(eps=float("nan")) == B.TK_ERR_VALUE
    # eps below 2^-126 would let the backward's fp32 row scale overflow
    for eps in (1e-39, 2.0 ** -127, 1e-300, 5e-324, float("inf")):
        assert fwd(eps=eps) == B.TK_ERR_VALUE, eps
        assert fwd(eps=eps, T=0) == B.TK_ERR_VALUE, eps
        assert bwd(eps=eps, T=0, ws=None, wsb=0) == B.TK_ERR_VALUE, eps
        assert noalloc(eps=eps) == B.TK_ERR_VALUE, eps
    assert fwd(eps=2.0 ** -126, T=0) == B.TK_SUCCESS
    assert bwd(eps=2.0 ** -126, T=0, ws=None, wsb=0) == B.TK_SUCCESS
    assert fwd(T=0, x=None) == B.TK_SUCCESS          # empty: nothing to do
    for name in ("x", "k", "v", "wh", "we", "out", "gate"):
        assert fwd(**{name: None}) == B.TK_ERR_NULL, name
    for name in ("x", "k", "v", "wh", "we", "out"):
        assert fwd(**{name: A16 + 8}) == B.TK_ERR_ALIGN, name
    assert fwd(gate=A16 + 2) == B.TK_ERR_ALIGN


def test_backward_argument_checks():
    assert bwd(T=-3) == B.TK_ERR_SHAPE
    assert bwd(H=20) == B.TK_ERR_ALIGN
    assert bwd(H=16384) == B.TK_ERR_UNSUPPORTED
    assert bwd(clamp=0.0) == B.TK_ERR_VALUE
    assert bwd(clamp=float("inf")) == B.TK_ERR_VALUE
    assert bwd(T=0, ws=None, wsb=0) == B.TK_SUCCESS
    for name in ("g", "x", "k", "v", "wh", "we", "dx", "dk", "dv", "ws"):
        assert bwd(**{name: None}) == B.TK_ERR_NULL, name
        assert bwd(**{name: A4}) == B.TK_ERR_ALIGN, name
    need = eg.tk_engram_bwd_workspace_bytes(4, 64)
    assert bwd(wsb=need - 4) == B.TK_ERR_WORKSPACE
    # the clamp is applied in fp32 and must round to a normal fp32 value
    for clamp in (1e-300, 1e-39, 1e-45, 1e39, -1e-4, float("nan")):
        assert bwd(clamp=clamp) == B.TK_ERR_VALUE, clamp
        assert bwd(clamp=clamp, T=0, ws=None, wsb=0) == B.TK_ERR_VALUE, clamp


def test_noalloc_backward_argument_checks():
    # only failing checks here: a call that passed them would launch
    assert noalloc(T=-3) == B.TK_ERR_SHAPE
    assert noalloc(H=20) == B.TK_ERR_ALIGN
    assert noalloc(H=16384) == B.TK_ERR_UNSUPPORTED
    assert noalloc(eps=-1.0) == B.TK_ERR_VALUE
    for clamp in (0.0, 1e-39, float("inf")):
        assert noalloc(clamp=clamp) == B.TK_ERR_VALUE, clamp
    for name in ("g", "x", "k", "v", "wh", "we", "dx", "dk", "dv", "dwh", "dwe"):
        assert noalloc(**{name: None}) == B.TK_ERR_NULL, name
        assert noalloc(**{name: A4}) == B.TK_ERR_ALIGN, name
    assert noalloc(T=0, dwh=None) == B.TK_ERR_NULL
    assert noalloc(T=0, dwe=A4) == B.TK_ERR_ALIGN
    # with T = 0 the reduction still runs (zeros into dwh, dwe) and reads the
    # weights, so they are checked too
    assert noalloc(T=0, wh=None) == B.TK_ERR_NULL
    assert noalloc(T=0, we=None) == B.TK_ERR_NULL
    assert noalloc(T=0, we=A4) == B.TK_ERR_ALIGN


def test_reduce_argument_checks():
    assert red(P=-1) == B.TK_ERR_SHAPE
    assert red(H=-8) == B.TK_ERR_SHAPE
    assert red(H=36) == B.TK_ERR_ALIGN
    assert red(H=9000) == B.TK_ERR_UNSUPPORTED
    assert red(P=B_MAX_PARTIALS + 1) == B.TK_ERR_UNSUPPORTED
    for name in ("ws", "wh", "we", "dwh", "dwe"):
        assert red(**{name: None}) == B.TK_ERR_NULL, name
        assert red(**{name: A4}) == B.TK_ERR_ALIGN, name


def test_copy_probe_argument_checks():
    L = eg.load_library()
    assert L.tk_engram_copy_probe(None, None, 0, None) == B.TK_SUCCESS
    assert L.tk_engram_copy_probe(None, A16, 64, None) == B.TK_ERR_NULL
    assert L.tk_engram_copy_probe(A16, A16, 40, None) == B.TK_ERR_ALIGN
    assert L.tk_engram_copy_probe(A4, A16, 64, None) == B.TK_ERR_ALIGN


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.ones(64)
    with pytest.raises(ValueError):
        eg.tk_engram_gate_fwd(x, x, x, w, w)


def test_probe_bindings_refuse_host_tensors():
    # a host pointer handed to a probe kernel would fault the GPU
    import torch
    a, b = torch.zeros(64, dtype=torch.int32), torch.zeros(64, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        eg.tk_engram_copy_probe(a, b)
    with pytest.raises(ValueError, match="GPU"):
        eg.tk_engram_stream_probe([a], [b])


def test_noalloc_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.ones(64)
    with pytest.raises(ValueError):
        eg.tk_engram_gate_bwd_reduce_noalloc(x, x, x, x, w, w)


def test_missing_library_raises(tmp_path):
    old = B._lib
    try:
        B._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            B.load_library(str(tmp_path / "nope.so"))
    finally:
        B._lib = old


def test_product_path_does_not_touch_the_oracle():
    # The library and its binding neither import nor link the oracle.
    pkg = os.path.join(ROOT, "engram_conditional_memory_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower(), f
    with open(eg.LIBRARY_PATH, "rb") as fh:
        assert b"oracle_" not in fh.read()


def test_autograd_wrapper_rejects_host_tensors():
    # the gate has no CPU implementation: host tensors are refused before any
    # library call
    import torch
    m = eg.EngramGate(64)
    x = torch.zeros(3, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        m(x, x, x)


def hsh(**kw):
    import numpy as np
    a = dict(tokens=A16, B=2, S=5, L=2, K=8, ngram=[2, 3], table=None, pad=0, out=A16)
    a.update(kw)
    L, K = a["L"], a["K"]
    ngram = np.ascontiguousarray(a["ngram"], dtype=np.int32)
    mult = np.ones((max(L, 1), max(K, 1), 4), dtype=np.uint64)
    table = (np.full((max(L, 1), max(K, 1)), 1021, dtype=np.uint32) if a["table"] is None
             else np.ascontiguousarray(a["table"], dtype=np.uint32))
    return eg.load_library().tk_engram_hash(
        a["tokens"], a["B"], a["S"], L, K, ngram.ctypes.data, mult.ctypes.data,
        table.ctypes.data, a["pad"], a["out"], None)


def test_hash_argument_checks():
    assert hsh(B=-1) == B.TK_ERR_SHAPE
    assert hsh(L=0, ngram=[2]) == B.TK_ERR_SHAPE
    assert hsh(K=0) == B.TK_ERR_SHAPE
    assert hsh(L=2, K=17) == B.TK_ERR_UNSUPPORTED           # 34 tables
    assert hsh(B=65536) == B.TK_ERR_UNSUPPORTED
    assert hsh(ngram=[2, 5]) == B.TK_ERR_VALUE
    assert hsh(ngram=[0, 3]) == B.TK_ERR_VALUE
    t = [[1021] * 8, [1021] * 7 + [0]]
    assert hsh(table=t) == B.TK_ERR_VALUE
    t = [[1021] * 8, [1021] * 7 + [(1 << 31) + 1]]
    assert hsh(table=t) == B.TK_ERR_VALUE
    assert hsh(B=0, tokens=None, out=None) == B.TK_SUCCESS
    assert hsh(S=0, tokens=None, out=None) == B.TK_SUCCESS
    assert hsh(tokens=None) == B.TK_ERR_NULL
    assert hsh(out=None) == B.TK_ERR_NULL
    assert hsh(tokens=A16 + 2) == B.TK_ERR_ALIGN
    assert hsh(out=A16 + 4) == B.TK_ERR_ALIGN


def gat(**kw):
    import numpy as np
    a = dict(idx=A16, T=4, Q=2, data=A16, R=100, d=64, off=[0, 50], rows=[50, 50], out=A16)
    a.update(kw)
    off = np.ascontiguousarray(a["off"], dtype=np.int64)
    rows = np.ascontiguousarray(a["rows"], dtype=np.uint32)
    return eg.load_library().tk_engram_gather(
        a["idx"], a["T"], a["Q"], a["data"], a["R"], a["d"], off.ctypes.data,
        rows.ctypes.data, a["out"], None)


def test_gather_argument_checks():
    assert gat(T=-1) == B.TK_ERR_SHAPE
    assert gat(Q=0) == B.TK_ERR_SHAPE
    assert gat(d=0) == B.TK_ERR_SHAPE
    assert gat(d=12) == B.TK_ERR_ALIGN
    assert gat(Q=33, off=[0] * 33, rows=[1] * 33) == B.TK_ERR_UNSUPPORTED
    assert gat(d=8200) == B.TK_ERR_UNSUPPORTED
    assert gat(off=[0, 51]) == B.TK_ERR_VALUE           # table 1 runs past R
    assert gat(off=[-1, 50]) == B.TK_ERR_VALUE
    assert gat(rows=[50, 51]) == B.TK_ERR_VALUE
    assert gat(T=0, idx=None, data=None, out=None) == B.TK_SUCCESS
    for name in ("idx", "data", "out"):
        assert gat(**{name: None}) == B.TK_ERR_NULL, name
    assert gat(idx=A16 + 2) == B.TK_ERR_ALIGN
    assert gat(data=A16 + 8) == B.TK_ERR_ALIGN
    assert gat(out=A4) == B.TK_ERR_ALIGN


def test_fused_weight_argument_checks():
    L = eg.load_library()
    assert L.tk_engram_fused_weight(A16, A16, A16, -1, None) == B.TK_ERR_SHAPE
    assert L.tk_engram_fused_weight(None, None, None, 0, None) == B.TK_SUCCESS
    assert L.tk_engram_fused_weight(None, A16, A16, 8, None) == B.TK_ERR_NULL
    assert L.tk_engram_fused_weight(A16, A16, A4, 8, None) == B.TK_ERR_ALIGN
    assert L.tk_engram_fused_weight(A16 + 2, A16, A16, 8, None) == B.TK_ERR_ALIGN


def test_stream_probe_argument_checks():
    import ctypes
    L = eg.load_library()
    two = (ctypes.c_void_p * 2)(A16, A16)
    bad = (ctypes.c_void_p * 2)(A16, A4)
    nul = (ctypes.c_void_p * 2)(A16, None)
    c = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert L.tk_engram_stream_probe(c(two), 0, c(two), 1, 64, None) == B.TK_ERR_SHAPE
    assert L.tk_engram_stream_probe(c(two), 1, c(two), 5, 64, None) == B.TK_ERR_SHAPE
    assert L.tk_engram_stream_probe(None, 1, c(two), 1, 64, None) == B.TK_ERR_NULL
    assert L.tk_engram_stream_probe(c(two), 2, c(two), 2, 0, None) == B.TK_SUCCESS
    assert L.tk_engram_stream_probe(c(two), 2, c(two), 2, 40, None) == B.TK_ERR_ALIGN
    assert L.tk_engram_stream_probe(c(bad), 2, c(two), 1, 64, None) == B.TK_ERR_ALIGN
    assert L.tk_engram_stream_probe(c(two), 1, c(nul), 2, 64, None) == B.TK_ERR_NULL
