"""The oracle's pins catch plausible mistakes.

Each mutant below is a copy of the oracle sources with one mistake planted
(a dropped term, a wrong sign, a transposed operand, a wrong index, ...).
The copy is built on the CPU, the pin tests run against it in a child
process, and at least one pin must fail. The regression snapshot of the tiny
workload is left out of these runs: it was written by the oracle itself, so
it would catch every mutant without showing that an independent pin does.
An unmutated copy built the same way must pass, so a failure is the
mistake's and not the harness's.
"""

import concurrent.futures
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ODIR = os.path.join(ROOT, "oracle")
SOURCES = ("engram_oracle.cpp", "compare.cpp", "engram_hash_oracle.cpp")
PIN_TESTS = ["tests/test_oracle.py", "tests/test_hash_oracle.py", "tests/test_compare.py"]

# (name, file, text as it stands, planted mistake). Each text must occur in
# the file; only its first occurrence is replaced.
MUTANTS = [
    ("eps outside the root", "engram_oracle.cpp",
     "*r = 1.0 / std::sqrt(*mean_sq + eps);", "*r = 1.0 / (std::sqrt(*mean_sq) + eps);"),
    ("RMSNorm weight dropped", "engram_oracle.cpp",
     "out[i] = row[i] * (*r) * w[i];", "out[i] = row[i] * (*r);"),
    ("mean over H - 1", "engram_oracle.cpp",
     "*mean_sq = sum_sq / (double)H;", "*mean_sq = sum_sq / (double)(H - 1);"),
    ("dot scaled by 1/H", "engram_oracle.cpp",
     "f.z = d * scalar;", "f.z = d / (double)H;"),
    ("scalar after signed_sqrt", "engram_oracle.cpp",
     "f.s = sign_of(f.z) * std::sqrt(std::fabs(f.z));",
     "f.s = sign_of(f.dot) * std::sqrt(std::fabs(f.dot)) * scalar;"),
    ("sign of z dropped", "engram_oracle.cpp",
     "f.s = sign_of(f.z) * std::sqrt(std::fabs(f.z));", "f.s = std::sqrt(std::fabs(f.z));"),
    ("sigmoid of -s", "engram_oracle.cpp",
     "f.gate = 1.0 / (1.0 + std::exp(-f.s));", "f.gate = 1.0 / (1.0 + std::exp(f.s));"),
    ("residual adds gate * x (fp64 path)", "engram_oracle.cpp",
     "out[t * H + i] = xr[i] + f.gate * vr[i];", "out[t * H + i] = xr[i] + f.gate * xr[i];"),
    ("dv without the gate", "engram_oracle.cpp",
     "dv[i] = f.gate * gout[i];", "dv[i] = gout[i];"),
    ("sigmoid derivative without (1 - gate)", "engram_oracle.cpp",
     "r.ds = dg * f.gate * (1.0 / (1.0 + std::exp(f.s)));", "r.ds = dg * f.gate;"),
    ("sigmoid derivative as gate squared", "engram_oracle.cpp",
     "r.ds = dg * f.gate * (1.0 / (1.0 + std::exp(f.s)));",
     "r.ds = dg * f.gate * (1.0 / (1.0 + std::exp(-f.s)));"),
    ("1 - gate formed by subtraction", "engram_oracle.cpp",
     "r.ds = dg * f.gate * (1.0 / (1.0 + std::exp(f.s)));",
     "r.ds = dg * f.gate * (1.0 - f.gate);"),
    ("clamp added instead of taken as a floor", "engram_oracle.cpp",
     "std::max(std::fabs(f.z), clamp)", "(std::fabs(f.z) + clamp)"),
    ("derivative clamp dropped", "engram_oracle.cpp",
     "std::max(std::fabs(f.z), clamp)", "std::max(std::fabs(f.z), 1e-300)"),
    ("backward multiplies by sqrt(H)", "engram_oracle.cpp",
     "r.dd = r.dz * scalar;", "r.dd = r.dz / scalar;"),
    ("operands of the dot transposed in the backward", "engram_oracle.cpp",
     "da[i] = r.dd * b[i];\n    db[i] = r.dd * a[i];",
     "da[i] = r.dd * a[i];\n    db[i] = r.dd * b[i];"),
    ("RMSNorm gradient term dropped from dx", "engram_oracle.cpp",
     " - rx3 * x[i] * sx / (double)H;", ";"),
    ("residual gradient dropped from dx", "engram_oracle.cpp",
     "dx[i] = gout[i] + f.r_x * wh[i] * da[i]", "dx[i] = f.r_x * wh[i] * da[i]"),
    ("dk takes wh", "engram_oracle.cpp",
     "dk[i] = f.r_k * we[i] * db[i]", "dk[i] = f.r_k * wh[i] * db[i]"),
    ("dwh from the k side", "engram_oracle.cpp",
     "dwh[i] += x[i] * f.r_x * da[i];", "dwh[i] += k[i] * f.r_k * db[i];"),
    ("r^3 as r^2", "engram_oracle.cpp",
     "const double rx3 = f.r_x * f.r_x * f.r_x;", "const double rx3 = f.r_x * f.r_x;"),
    ("bf16 widened with a wrong shift", "engram_oracle.cpp",
     "uint32_t u = ((uint32_t)bits) << 16;", "uint32_t u = ((uint32_t)bits) << 15;"),
    ("rounding ties away from even", "engram_oracle.cpp",
     "(dropped > half || (dropped == half && (keep & 1)))", "(dropped >= half)"),
    ("rounding to the wrong kept width", "engram_oracle.cpp",
     "uint64_t keep = frac >> 45;", "uint64_t keep = frac >> 44;"),
    ("overflow to infinity from 2^129 instead of 2^128", "engram_oracle.cpp",
     "if (e > 127) return sbit | 0x7F80;", "if (e > 128) return sbit | 0x7F80;"),
    ("rounding past the largest finite value saturates", "engram_oracle.cpp",
     "if (biased >= 255) return (uint16_t)((sign << 15) | 0x7F80);",
     "if (biased >= 255) return (uint16_t)((sign << 15) | 0x7F7F);"),
    ("subnormal quantum 2^-134 instead of 2^-133", "engram_oracle.cpp",
     "const double units = mag * 0x1p133;", "const double units = mag * 0x1p134;"),
    ("subnormal ties rounded away from even", "engram_oracle.cpp",
     "(frac > 0.5 || (frac == 0.5 && std::fmod(lo, 2.0) != 0.0))", "(frac >= 0.5)"),
    ("hash sums the products instead of XOR", "engram_hash_oracle.cpp",
     "h ^= (uint64_t)tok * a[i];", "h += (uint64_t)tok * a[i];"),
    ("hash window one position short at the start", "engram_hash_oracle.cpp",
     "const uint32_t tok = p >= 0 ? (uint32_t)seq[p] : pad;",
     "const uint32_t tok = p > 0 ? (uint32_t)seq[p] : pad;"),
    ("hash truncated to 32 bits before the modulus", "engram_hash_oracle.cpp",
     "(int32_t)(h % (uint64_t)table_size[l * K + j])",
     "(int32_t)((uint32_t)h % (uint64_t)table_size[l * K + j])"),
    ("hash multipliers of the wrong position", "engram_hash_oracle.cpp",
     "h ^= (uint64_t)tok * a[i];", "h ^= (uint64_t)tok * a[n - 1 - i];"),
    ("ulp distance without the sign", "compare.cpp",
     "return (bits & 0x8000) ? -mag : mag;", "return mag;"),
]


def build_copy(tmp, name, mutation):
    """Copy the oracle sources into `tmp`, plant `mutation` (file, old, new)
    if given, and build the library there; returns its path."""
    os.makedirs(tmp, exist_ok=True)
    paths = []
    for src in SOURCES:
        with open(os.path.join(ODIR, src)) as f:
            text = f.read()
        if mutation and mutation[0] == src:
            old, new = mutation[1], mutation[2]
            assert old in text, f"{name}: text not found in {src}"
            text = text.replace(old, new, 1)
        p = os.path.join(tmp, src)
        with open(p, "w") as f:
            f.write(text)
        paths.append(p)
    lib = os.path.join(tmp, "liboracle.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
                    "-pthread", *paths, "-o", lib], check=True, capture_output=True)
    return lib


def run_pins(lib):
    env = dict(os.environ)
    env[oracle.LIB_OVERRIDE_ENV] = lib
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([sys.executable, "-m", "pytest", *PIN_TESTS, "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu", "-k", "not snapshot"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    failed = [ln.split(" ")[1] for ln in r.stdout.splitlines() if ln.startswith("FAILED ")]
    return r.returncode, failed, r.stdout[-2000:]


@pytest.mark.timeout(900)
def test_every_planted_mistake_fails_a_pin(tmp_path):
    rc, failed, out = run_pins(build_copy(str(tmp_path / "clean"), "clean", None))
    assert rc == 0, "the unmutated copy must pass its pins:\n" + out

    def one(i):
        name, src, old, new = MUTANTS[i]
        lib = build_copy(str(tmp_path / f"m{i}"), name, (src, old, new))
        return (name,) + run_pins(lib)

    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(one, range(len(MUTANTS))))
    survivors = []
    for name, rc, failed, out in results:
        print(f"{name}: {'caught by ' + failed[0] if rc == 1 and failed else 'rc ' + str(rc)}")
        # rc 1 is "some test failed"; a crash of the child also counts as caught
        if rc == 0 or rc == 5:
            survivors.append(name)
    assert not survivors, f"mutants that no pin catches: {survivors}"
