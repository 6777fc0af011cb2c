"""Python handle on the fp64 Engram gate oracle (``engram_oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The GPU library never imports,
links or calls it, and it imports nothing from the GPU library.

What it computes is the gate of the zhichai.net TileKernels page, section
"5. Engram" (gate formula), and its chain-rule backward; the readings taken
where that page is silent are listed at the top of ``engram_oracle.cpp``.
The same section's N-gram hash (engram_hash) is in ``engram_hash_oracle.cpp``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "engram_oracle.cpp")
_SRC_CMP = os.path.join(_HERE, "compare.cpp")
_SRC_HASH = os.path.join(_HERE, "engram_hash_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation test plants mistakes in a copy of the sources and points this
# variable at the copy's library, to show that the pins catch each mistake.
LIB_OVERRIDE_ENV = "TK_ENGRAM_ORACLE_LIB"

EPS = 1e-6          # RMSNorm epsilon used throughout (the pages give none)
CLAMP = 1e-4        # lower clamp of |z| in the signed-sqrt derivative


def build(verbose: bool = False) -> str:
    """Compile the oracle with g++ (no fast-math, no FMA contraction)."""
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", _SRC, _SRC_CMP, _SRC_HASH, "-o", _LIB]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get(LIB_OVERRIDE_ENV) or _LIB
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, i64, dbl, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
        L.oracle_fwd_f64.argtypes = [vp, vp, vp, vp, vp, i64, i64, dbl, vp, vp, vp]
        L.oracle_bwd_f64.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, dbl, dbl,
                                     vp, vp, vp, vp, vp, vp]
        L.oracle_fwd_bf16.argtypes = [vp, vp, vp, vp, vp, i64, i64, dbl, vp, vp, vp, i32]
        L.oracle_bwd_bf16.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, dbl, dbl,
                                      vp, vp, vp, vp, vp, vp, i32]
        L.oracle_round_bf16.argtypes = [vp, i64, vp]
        L.oracle_compare_bf16.argtypes = [vp, vp, i64, i64, vp, vp, i32]
        L.oracle_check_out.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp, i32]
        L.oracle_engram_hash.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp,
                                         ctypes.c_uint32, vp]
        for n in ("oracle_fwd_f64", "oracle_bwd_f64", "oracle_fwd_bf16",
                  "oracle_bwd_bf16", "oracle_round_bf16", "oracle_compare_bf16",
                  "oracle_check_out", "oracle_engram_hash"):
            getattr(L, n).restype = None
        L.oracle_fwd_stats_width.restype = i32
        L.oracle_bwd_stats_width.restype = i32
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need C-contiguous"
    return a.ctypes.data


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---- fp64 inputs ------------------------------------------------------------

def fwd_f64(x, k, v, wh, we, eps=EPS):
    """Forward on fp64 arrays.  Returns (out [T,H], gate [T], stats [T,8]) with
    stats columns mean(x^2), mean(k^2), r_x, r_k, d, z, s, gate."""
    x, k, v, wh, we = map(_f64, (x, k, v, wh, we))
    T, H = x.shape
    out = np.empty((T, H)); gate = np.empty(T); st = np.empty((T, 8))
    lib().oracle_fwd_f64(_p(x), _p(k), _p(v), _p(wh), _p(we), T, H, eps,
                         _p(out), _p(gate), _p(st))
    return out, gate, st


def bwd_f64(gout, x, k, v, wh, we, eps=EPS, clamp=CLAMP):
    """Backward on fp64 arrays.  Returns (dx, dk, dv, dwh, dwe, stats [T,4])
    with stats columns dgate, ds, dz, dd."""
    gout, x, k, v, wh, we = map(_f64, (gout, x, k, v, wh, we))
    T, H = x.shape
    dx = np.empty((T, H)); dk = np.empty((T, H)); dv = np.empty((T, H))
    dwh = np.empty(H); dwe = np.empty(H); st = np.empty((T, 4))
    lib().oracle_bwd_f64(_p(gout), _p(x), _p(k), _p(v), _p(wh), _p(we), T, H, eps,
                         clamp, _p(dx), _p(dk), _p(dv), _p(dwh), _p(dwe), _p(st))
    return dx, dk, dv, dwh, dwe, st


# ---- bf16 inputs (uint16 bit patterns), multithreaded -------------------------

def fwd_bf16(x, k, v, wh, we, eps=EPS, want_out=True, threads=None):
    """Forward over bf16 rows.  Returns (out fp64 [rows,H] or None, gate, z)."""
    rows, H = x.shape
    for a in (x, k, v):
        assert a.dtype == np.uint16 and a.shape == (rows, H) and a.flags["C_CONTIGUOUS"]
    wh = np.ascontiguousarray(wh, dtype=np.float32)
    we = np.ascontiguousarray(we, dtype=np.float32)
    out = np.empty((rows, H)) if want_out else None
    gate = np.empty(rows); z = np.empty(rows)
    lib().oracle_fwd_bf16(_p(x), _p(k), _p(v), _p(wh), _p(we), rows, H, eps,
                          _p(out), _p(gate), _p(z), threads or default_threads())
    return out, gate, z


def bwd_bf16(gout, x, k, v, wh, we, eps=EPS, clamp=CLAMP, want_grads=True,
             threads=None):
    """Backward over bf16 rows.  Returns (dx, dk, dv or Nones, dwh, dwe, dd)."""
    rows, H = x.shape
    for a in (gout, x, k, v):
        assert a.dtype == np.uint16 and a.shape == (rows, H) and a.flags["C_CONTIGUOUS"]
    wh = np.ascontiguousarray(wh, dtype=np.float32)
    we = np.ascontiguousarray(we, dtype=np.float32)
    if want_grads:
        dx = np.empty((rows, H)); dk = np.empty((rows, H)); dv = np.empty((rows, H))
    else:
        dx = dk = dv = None
    dwh = np.empty(H); dwe = np.empty(H); dd = np.empty(rows)
    lib().oracle_bwd_bf16(_p(gout), _p(x), _p(k), _p(v), _p(wh), _p(we), rows, H,
                          eps, clamp, _p(dx), _p(dk), _p(dv), _p(dwh), _p(dwe),
                          _p(dd), threads or default_threads())
    return dx, dk, dv, dwh, dwe, dd


def round_bf16(a) -> np.ndarray:
    """fp64 -> bf16 bit patterns, nearest-even."""
    a = _f64(a)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_round_bf16(_p(a), a.size, _p(out))
    return out


def bf16_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- comparison statistics (test infrastructure) -------------------------------

class BF16Stats:
    """Streaming error statistics of bf16 GPU results against the oracle's fp64
    values rounded to bf16, split by row class (0 = regular rows)."""

    CLASSES = 4

    def __init__(self):
        self.acc = np.zeros(self.CLASSES * 6)

    def add(self, gpu_bits, ref, row_class=None, threads=None):
        rows, H = ref.shape
        assert gpu_bits.shape == (rows, H) and gpu_bits.dtype == np.uint16
        gpu_bits = np.ascontiguousarray(gpu_bits)
        ref = np.ascontiguousarray(ref, dtype=np.float64)
        rc = None if row_class is None else np.ascontiguousarray(row_class, dtype=np.uint8)
        lib().oracle_compare_bf16(_p(gpu_bits), _p(ref), rows, H, _p(rc), _p(self.acc),
                                  threads or default_threads())

    def _cls(self, classes):
        a = self.acc.reshape(self.CLASSES, 6)
        return a[list(classes)]

    def rel_l2(self, classes=(0, 1, 2, 3)):
        a = self._cls(classes)
        den = a[:, 1].sum()
        return float(np.sqrt(a[:, 0].sum() / den)) if den > 0 else float(a[:, 0].sum() > 0)

    def max_ulp(self, classes=(0, 1, 2, 3)):
        return float(self._cls(classes)[:, 2].max())

    def count_over_1ulp(self, classes=(0, 1, 2, 3)):
        return int(self._cls(classes)[:, 3].sum())

    def max_row_rel(self, classes=(0, 1, 2, 3)):
        return float(self._cls(classes)[:, 4].max())

    def nonfinite(self):
        return int(self.acc.reshape(self.CLASSES, 6)[:, 5].sum())


def check_out(gpu_bits, ref, x_bits, v_bits, gate, res=None, threads=None):
    """Accumulate the forward-output check; returns res = [max ulp, n > 1 ulp,
    n passing by the cancellation bound, n failing]."""
    rows, H = ref.shape
    res = np.zeros(4) if res is None else res
    arrs = [np.ascontiguousarray(a) for a in (gpu_bits, x_bits, v_bits)]
    ref = np.ascontiguousarray(ref, dtype=np.float64)
    gate = np.ascontiguousarray(gate, dtype=np.float64)
    lib().oracle_check_out(_p(arrs[0]), _p(ref), _p(arrs[1]), _p(arrs[2]), _p(gate),
                           rows, H, _p(res), threads or default_threads())
    return res


# ---- N-gram hash (engram_hash_oracle.cpp) -------------------------------------

def engram_hash(tokens, ngram, mult, table_size, pad):
    """Table indices int32 [B, S, L, K] of the N-gram hash.

    tokens int32 [B, S]; ngram [L] N-gram orders (1..4); mult uint64 [L, K, 4]
    multipliers (entries past n_l unused); table_size uint32 [L, K]; pad the
    token id read before the start of a sequence."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    assert tokens.ndim == 2
    B, S = tokens.shape
    ngram = np.ascontiguousarray(ngram, dtype=np.int32)
    mult = np.ascontiguousarray(mult, dtype=np.uint64)
    table_size = np.ascontiguousarray(table_size, dtype=np.uint32)
    L, K = table_size.shape
    assert ngram.shape == (L,) and mult.shape == (L, K, 4)
    assert np.all((ngram >= 1) & (ngram <= 4)) and np.all(table_size >= 1)
    out = np.empty((B, S, L, K), dtype=np.int32)
    lib().oracle_engram_hash(_p(tokens), B, S, L, K, _p(ngram), _p(mult), _p(table_size),
                             int(pad) & 0xFFFFFFFF, _p(out))
    return out


# ---- hashed multi-table gather ---------------------------------------------------

def engram_gather(idx, table_data, row_offset, rows):
    """out [T, Q, d] with out[t, q] = table_data[row_offset[q] + idx[t, q]] when
    0 <= idx[t, q] < rows[q], else a zero row (bf16 bit patterns)."""
    idx = np.asarray(idx, dtype=np.int64)
    T, Q = idx.shape
    row_offset = np.asarray(row_offset, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    valid = (idx >= 0) & (idx < rows[None, :])
    src = np.where(valid, row_offset[None, :] + idx, 0)
    out = table_data[src]                       # library gather
    out[~valid] = 0
    return out


# ---- fused RMSNorm weight ---------------------------------------------------------

def fused_weight(wh, we):
    """w = wh * we for fp32 inputs, in fp64 (the product of two 24-bit
    significands has at most 48 bits, so it is exact in fp64)."""
    return np.asarray(wh, dtype=np.float32).astype(np.float64) * \
        np.asarray(we, dtype=np.float32).astype(np.float64)

