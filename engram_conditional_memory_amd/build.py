"""Build libtk_engram.so, the HIP library behind include/tk_engram.h, for gfx950."""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "engram_gate.hip"),
        os.path.join(PKG, "csrc", "engram_hash.hip"),
        os.path.join(PKG, "csrc", "engram_gather.hip"),
        os.path.join(PKG, "csrc", "engram_status.cpp")]
LIB = os.path.join(PKG, "libtk_engram.so")
INCLUDE = os.path.join(ROOT, "include")


def hipcc_command(out: str = LIB) -> list[str]:
    return [
        "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 instructions stay off on this device
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, *SRCS, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi", "gate_c_example.cpp")
EXAMPLE = os.path.join(ROOT, "tests", "c_abi", "gate_c_example")


def build_example(verbose: bool = False) -> str:
    """Build the host-only C++ program that calls the library through its C ABI
    (linked against the in-tree libtk_engram.so by relative rpath)."""
    cmd = ["hipcc", "-O2", "-std=c++17", "-I", INCLUDE, EXAMPLE_SRC, "-L", PKG, "-ltk_engram",
           "-Wl,-rpath,$ORIGIN/../../engram_conditional_memory_amd", "-o", EXAMPLE]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{r.stdout}\n{r.stderr}")
    return EXAMPLE


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_example(verbose=True))
