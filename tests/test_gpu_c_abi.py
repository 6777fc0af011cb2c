"""The library used from plain host C++ through include/tk_engram.h alone
(tests/c_abi/gate_c_example.cpp, built by __graft_entry__.build())."""

import os
import subprocess

import pytest

from engram_conditional_memory_amd.build import EXAMPLE

pytestmark = pytest.mark.gpu


def test_c_abi_example_program(cuda_device):
    if not os.path.exists(EXAMPLE):
        pytest.fail(f"{EXAMPLE} is missing: run __graft_entry__.build()")
    r = subprocess.run([EXAMPLE], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi example ok" in r.stdout
