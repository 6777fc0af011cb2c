"""Seeded synthetic inputs for the Engram gate workloads.

The gate itself is described on the zhichai.net TileKernels page, section
"5. Engram" (gate formula): per token a hidden row x, a key row k and a value
row v, all of width H, plus two per-channel RMSNorm weights wh and we.  The
pages print no data, so every workload here is drawn from a counter-based
generator (Philox-4x32-10) with a fixed seed, with the shapes of the pages'
example ([batch, seq_len, hidden_dim] with hidden_dim in {4096, 7168}).

This module holds none of the gate's arithmetic.  It produces host arrays:
bf16 tensors as uint16 bit patterns, fp32 weights as float32.  Both the fp64
oracle (``oracle/``) and the GPU library consume the identical bytes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.cpp")
_LIB = os.path.join(_HERE, "libsynth.so")

# Stream ids: one independent Philox stream per tensor or per-row draw.
STREAM_X, STREAM_K, STREAM_V, STREAM_GOUT = 1, 2, 3, 4
STREAM_WH, STREAM_WE = 5, 6
STREAM_RHO, STREAM_KNOISE = 7, 8
STREAM_MASK = {"x": 9, "k": 10, "v": 11}
STREAM_TOKENS = 12


def build(verbose: bool = False) -> str:
    """Compile the generator with g++ into ``synth/libsynth.so``."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
           _SRC, "-o", _LIB]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        u64, u32, i64, i32, dbl = (ctypes.c_uint64, ctypes.c_uint32,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_double)
        vp = ctypes.c_void_p
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_round_bf16.argtypes = [vp, i64, vp]
        L.synth_normal_bf16.argtypes = [u64, u32, i64, i64, dbl, vp, i32]
        L.synth_normal_f32.argtypes = [u64, u32, i64, i64, dbl, dbl, vp]
        L.synth_uniform_pm1.argtypes = [u64, u32, i64, i64, vp]
        L.synth_row_keys.argtypes = [u64, u32, i64, vp]
        L.synth_correlated_bf16.argtypes = [u64, u32, vp, vp, i64, i64, i64, vp, i32]
        L.synth_student_t3_bf16.argtypes = [u64, u32, i64, i64, i64, vp, vp, i32]
        for name in ("synth_philox4x32_10", "synth_round_bf16", "synth_normal_bf16",
                     "synth_normal_f32", "synth_uniform_pm1", "synth_row_keys",
                     "synth_correlated_bf16", "synth_student_t3_bf16"):
            getattr(L, name).restype = None
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---- primitive draws -------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().synth_round_bf16(_p(v), v.size, _p(out))
    return out


def normal_bf16(seed, stream, shape, e0=0, scale=1.0, threads=None) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_bf16(seed, stream, e0, out.size, scale, _p(out),
                            threads or default_threads())
    return out


def normal_f32(seed, stream, n, mean=0.0, std=1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, stream, 0, n, mean, std, _p(out))
    return out


def uniform_pm1(seed, stream, n, e0=0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_pm1(seed, stream, e0, n, _p(out))
    return out


def row_keys(seed, stream, n) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_row_keys(seed, stream, n, _p(out))
    return out


def correlated_bf16(seed, x_bits, rho, t0=0, threads=None) -> np.ndarray:
    rows, H = x_bits.shape
    out = np.empty_like(x_bits)
    lib().synth_correlated_bf16(seed, STREAM_KNOISE, _p(x_bits), _p(rho), t0, rows,
                                H, _p(out), threads or default_threads())
    return out


def student_t3_bf16(seed, stream, rows, H, row_scale, t0=0, threads=None) -> np.ndarray:
    row_scale = np.ascontiguousarray(row_scale, dtype=np.float64)
    assert row_scale.shape == (rows,)
    out = np.empty((rows, H), dtype=np.uint16)
    lib().synth_student_t3_bf16(seed, stream, t0, rows, H, _p(row_scale), _p(out),
                                threads or default_threads())
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (for test-side statistics only)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- the five workloads ----------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    kind: str          # "normal", "correlated" or "stress"
    fwd_only: bool
    describe: str


CONFIGS = {
    1: Config("tiny", 64, 256, "normal", False,
              "T=64 tokens, H=256, x,k,v ~ N(0,1) bf16, wh,we = 1+0.1N(0,1) fp32, "
              "grad_out ~ N(0,1), eps=1e-6, seed 0"),
    2: Config("fwd_b2s512_h4096", 2 * 512, 4096, "normal", True,
              "forward only, batch 2 x seq 512 = 1024 tokens, H=4096, x,k,v ~ N(0,1)"),
    3: Config("fwdbwd_b4s4096_h4096", 4 * 4096, 4096, "correlated", False,
              "fwd+bwd, batch 4 x seq 4096 = 16384 tokens, H=4096, x,v ~ N(0,1), "
              "k = rho x + sqrt(1-rho^2) N(0,1), rho ~ U[-1,1] per token"),
    4: Config("fwdbwd_b8s4096_h7168", 8 * 4096, 7168, "correlated", False,
              "fwd+bwd, batch 8 x seq 4096 = 32768 tokens, H=7168, correlated k"),
    5: Config("stress_t65537_h7168", 65537, 7168, "stress", False,
              "stress fwd+bwd, T=65537 (ragged), H=7168, x,k,v ~ Student-t(3), "
              "0.1% rows x1e3 and 0.1% rows all-zero per tensor"),
}


def stress_row_scales(seed: int, T: int, tensor: str) -> np.ndarray:
    """Per-row scale for a stress tensor: 1, 1e3 (round(0.001 T) rows) or 0
    (another round(0.001 T) rows, disjoint), rows picked by sorting Philox keys."""
    n = int(round(0.001 * T))
    order = np.argsort(row_keys(seed, STREAM_MASK[tensor], T), kind="stable")
    s = np.ones(T, dtype=np.float64)
    s[order[:n]] = 1e3
    s[order[n:2 * n]] = 0.0
    return s


def make_inputs(cfg: int | Config, seed: int = 0, rows: tuple[int, int] | None = None,
                threads: int | None = None, with_grad: bool = True) -> dict:
    """Host arrays for a workload, optionally only rows [r0, r1) of it.

    Returns x, k, v (and grad_out) as uint16 bf16 bits of shape [rows, H],
    wh and we as float32 [H], plus T, H and r0."""
    c = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    T, H = c.T, c.H
    r0, r1 = rows if rows is not None else (0, T)
    assert 0 <= r0 <= r1 <= T
    n = r1 - r0
    e0 = r0 * H
    th = threads or default_threads()
    out = {"T": T, "H": H, "r0": r0, "config": c}
    out["wh"] = normal_f32(seed, STREAM_WH, H, 1.0, 0.1)
    out["we"] = normal_f32(seed, STREAM_WE, H, 1.0, 0.1)
    if c.kind == "stress":
        for name, stream in (("x", STREAM_X), ("k", STREAM_K), ("v", STREAM_V)):
            s = stress_row_scales(seed, T, name)[r0:r1]
            out[name] = student_t3_bf16(seed, stream, n, H, s, t0=r0, threads=th)
    else:
        out["x"] = normal_bf16(seed, STREAM_X, (n, H), e0=e0, threads=th)
        out["v"] = normal_bf16(seed, STREAM_V, (n, H), e0=e0, threads=th)
        if c.kind == "correlated":
            rho = uniform_pm1(seed, STREAM_RHO, n, e0=r0)
            out["rho"] = rho
            out["k"] = correlated_bf16(seed, out["x"], rho, t0=r0, threads=th)
        else:
            out["k"] = normal_bf16(seed, STREAM_K, (n, H), e0=e0, threads=th)
    if with_grad:
        out["grad_out"] = normal_bf16(seed, STREAM_GOUT, (n, H), e0=e0, threads=th)
    return out


# ---- N-gram hash workloads ---------------------------------------------------

_MASK64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> list:
    """n outputs of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) from `seed`."""
    out = []
    state = seed & _MASK64
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def _is_prime(n: int) -> bool:
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    f = 3
    while f * f <= n:
        if n % f == 0:
            return False
        f += 2
    return True


def primes_below(limit: int, count: int) -> list:
    """The `count` largest primes below `limit`, descending."""
    out = []
    n = limit - 1
    while len(out) < count:
        if _is_prime(n):
            out.append(n)
        n -= 1
    return out


@dataclass(frozen=True)
class HashConfig:
    name: str
    B: int
    S: int
    ngram: tuple         # N-gram order of each layer
    tables: int          # tables per layer
    table_rows: int      # table sizes are distinct primes just below this
    vocab: int
    describe: str
    zipf: float = 0.0    # 0: ids uniform over the vocabulary; s > 0: Zipf(s) frequencies


HASH_CONFIGS = {
    "tiny": HashConfig("hash_tiny", 3, 37, (2, 3), 8, 1021, 1000,
                       "3 sequences of 37 tokens, 2-gram and 3-gram layers, 8 tables each"),
    "b8s4096": HashConfig("hash_b8s4096", 8, 4096, (2, 3), 8, 1 << 19, 129280,
                          "batch 8 x seq 4096 = 32768 tokens (the H=7168 gate workload), "
                          "2-gram and 3-gram layers, 8 tables each of ~2^19 rows"),
    "b8s4096_zipf": HashConfig("hash_b8s4096_zipf", 8, 4096, (2, 3), 8, 1 << 19, 129280,
                               "batch 8 x seq 4096 = 32768 tokens whose frequencies follow "
                               "Zipf(1) over the vocabulary, as word frequencies in text do; "
                               "same layers and tables", zipf=1.0),
    "b64s4096": HashConfig("hash_b64s4096", 64, 4096, (2, 3), 8, 1 << 19, 129280,
                           "batch 64 x seq 4096 = 262144 tokens, same layers and tables"),
    "b1024s4096": HashConfig("hash_b1024s4096", 1024, 4096, (2, 3), 8, 1 << 19, 129280,
                             "batch 1024 x seq 4096 = 4194304 tokens (throughput), "
                             "same layers and tables"),
}


def hash_params(cfg: HashConfig, seed: int = 0) -> dict:
    """Multipliers (odd, SplitMix64 from the seed) and prime table sizes for a
    hash workload; the pad id is the vocabulary size (one past the last id)."""
    L, K = len(cfg.ngram), cfg.tables
    raw = splitmix64(seed ^ 0x5EEDBA5E, L * K * 4)
    mult = np.array([v | 1 for v in raw], dtype=np.uint64).reshape(L, K, 4)
    sizes = np.array(primes_below(cfg.table_rows, L * K), dtype=np.uint32).reshape(L, K)
    return {"ngram": np.array(cfg.ngram, dtype=np.int32), "mult": mult,
            "table_size": sizes, "pad": cfg.vocab}


# Zipf ranks map to ids through r -> (r * ZIPF_ID_STRIDE + ZIPF_ID_SHIFT) mod
# vocab, a bijection whenever the stride is coprime with the vocabulary size,
# so the frequent tokens are spread over the id range instead of being the
# smallest ids.
ZIPF_ID_STRIDE = 7919
ZIPF_ID_SHIFT = 17


def zipf_ranks(u01: np.ndarray, vocab: int, s: float) -> np.ndarray:
    """Ranks in [0, vocab) with P(rank = r) proportional to (r + 1)^-s, by
    inverting the cumulative distribution at the uniforms u01 in [0, 1)."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** -s
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    return np.minimum(np.searchsorted(cdf, u01, side="right"), vocab - 1)


def zipf_rank_to_id(rank: np.ndarray, vocab: int) -> np.ndarray:
    assert np.gcd(ZIPF_ID_STRIDE, vocab) == 1
    return (np.asarray(rank, dtype=np.int64) * ZIPF_ID_STRIDE + ZIPF_ID_SHIFT) % vocab


def hash_tokens(cfg: HashConfig, seed: int = 0) -> np.ndarray:
    """Token ids int32 [B, S] from the Philox stream: uniform over the
    vocabulary, or with Zipf(cfg.zipf) frequencies when cfg.zipf > 0."""
    n = cfg.B * cfg.S
    u01 = (uniform_pm1(seed, STREAM_TOKENS, n) + 1.0) * 0.5     # in [0, 1)
    if cfg.zipf > 0:
        ids = zipf_rank_to_id(zipf_ranks(u01, cfg.vocab, cfg.zipf), cfg.vocab)
    else:
        ids = np.floor(u01 * cfg.vocab).astype(np.int64)
    return np.clip(ids, 0, cfg.vocab - 1).astype(np.int32).reshape(cfg.B, cfg.S)


# ---- embedding tables for the hashed gather -----------------------------------

def table_bits_np(q: int, rows, d: int) -> np.ndarray:
    """bf16 bit patterns of rows `rows` (int array) of table q, [len(rows), d].

    Each value is a finite bf16 in +-[1, 2) whose bits come from an integer
    mix of (table, row, column), so every row of every table is distinct and
    can be recomputed anywhere from its coordinates."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    cols = np.arange(d, dtype=np.uint64).reshape(1, -1)
    h = (rows * np.uint64(0x9E3779B1) + cols * np.uint64(0x85EBCA77)
         + np.uint64(q) * np.uint64(0xC2B2AE3D)) & np.uint64(0xFFFFFFFF)
    h ^= h >> np.uint64(15)
    h = (h * np.uint64(0x2C1B3C6D)) & np.uint64(0xFFFFFFFF)
    h ^= h >> np.uint64(12)
    sign = (h >> np.uint64(20)) & np.uint64(1)
    return ((sign << np.uint64(15)) | np.uint64(0x3F80) | (h & np.uint64(0x7F))).astype(np.uint16)


def fill_table_bits_torch(data, q: int, row0: int, rows: int, d: int):
    """The same pattern as table_bits_np, written into rows [row0, row0 + rows)
    of the bf16 tensor `data` [R, d] with torch integer ops on its device."""
    import torch
    dev = data.device
    r = torch.arange(rows, dtype=torch.int64, device=dev).view(-1, 1)
    c = torch.arange(d, dtype=torch.int64, device=dev).view(1, -1)
    m32 = 0xFFFFFFFF
    h = (r * 0x9E3779B1 + c * 0x85EBCA77 + q * 0xC2B2AE3D) & m32
    h = h ^ (h >> 15)
    h = (h * 0x2C1B3C6D) & m32
    h = h ^ (h >> 12)
    bits = (((h >> 20) & 1) << 15) | 0x3F80 | (h & 0x7F)
    bits = torch.where(bits >= 0x8000, bits - 0x10000, bits).to(torch.int16)
    data[row0:row0 + rows].view(torch.int16).copy_(bits)


@dataclass(frozen=True)
class GatherConfig:
    name: str
    T: int
    tables: int
    rows: int            # rows per table
    d: int               # row width (bf16)
    describe: str


GATHER_CONFIGS = {
    "tiny": GatherConfig("gather_tiny", 40, 16, 1021, 24,
                         "40 tokens x 16 tables of 1021 rows x 24"),
    "t32768_d448": GatherConfig("gather_t32768_d448", 32768, 16, 1 << 19, 448,
                                "32768 tokens x 16 tables (2 layers x 8) of 2^19 rows x 448 "
                                "bf16 (16 x 448 = 7168 = H)"),
}

