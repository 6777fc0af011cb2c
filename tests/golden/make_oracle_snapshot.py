"""Write config1_oracle_snapshot.txt: the fp64 oracle's outputs on the tiny
workload (T=64, H=256, seed 0), as a regression record of the oracle itself.

The pages print no worked example of the Engram gate, so no value here comes
from them; every value is produced by ``oracle/`` on inputs from ``synth``.
Run from the repository root:  python tests/golden/make_oracle_snapshot.py
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config1_oracle_snapshot.txt")


def main():
    d = synth.make_inputs(1)
    _, gate, z = oracle.fwd_bf16(d["x"], d["k"], d["v"], d["wh"], d["we"], threads=1)
    dx, dk, dv, dwh, dwe, dd = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"],
                                               d["wh"], d["we"], threads=1)
    with open(OUT, "w") as f:
        f.write("# fp64 oracle on the tiny workload (T=64, H=256, seed 0, eps=1e-6, clamp=1e-4)\n")
        f.write("# written by tests/golden/make_oracle_snapshot.py (calls only oracle/ and synth)\n")
        f.write("# columns: row gate z dd sum(dx) sum(dk) sum(dv)\n")
        for t in range(64):
            f.write(f"row {t} {gate[t]:.17g} {z[t]:.17g} {dd[t]:.17g} "
                    f"{dx[t].sum():.17g} {dk[t].sum():.17g} {dv[t].sum():.17g}\n")
        f.write("# columns: col dwh dwe (every 8th column)\n")
        for i in range(0, 256, 8):
            f.write(f"col {i} {dwh[i]:.17g} {dwe[i]:.17g}\n")


if __name__ == "__main__":
    main()
