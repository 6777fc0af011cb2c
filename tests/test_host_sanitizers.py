"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

The oracle, comparison, hash-oracle and generator C++ are built with g++ and
-fsanitize=address,undefined and driven on small inputs; the C ABI's
argument checks are built from the library sources with hipcc, sanitizers on
the host half only, and driven without a GPU (every call returns before any
device work). Any invalid access or undefined behaviour fails the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_oracle")
    srcs = [os.path.join(HERE, "host_oracle_main.cpp"),
            os.path.join(ROOT, "oracle", "engram_oracle.cpp"),
            os.path.join(ROOT, "oracle", "compare.cpp"),
            os.path.join(ROOT, "oracle", "engram_hash_oracle.cpp"),
            os.path.join(ROOT, "synth", "synth.cpp")]
    run(["g++", "-O1", "-g", "-std=c++17", "-pthread", *SAN, *srcs, "-o", exe])
    out = run([exe], env=ENV)
    assert "host oracle program ok" in out


def test_c_abi_checks_under_asan_ubsan(tmp_path):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_abi")
    pkg = os.path.join(ROOT, "engram_conditional_memory_amd", "csrc")
    srcs = [os.path.join(pkg, f) for f in ("engram_gate.hip", "engram_hash.hip",
                                           "engram_gather.hip", "engram_status.cpp")]
    host_san = []
    for flag in SAN:
        host_san += ["-Xarch_host", flag]
    run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
         "-I", os.path.join(ROOT, "include"), *srcs,
         os.path.join(HERE, "host_abi_main.cpp"), "-o", exe])
    out = run([exe], env=ENV)
    assert "host ABI program ok" in out
