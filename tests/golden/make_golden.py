"""Writes tests/golden/tiny_oracle.txt from the fp64 oracle alone (a regression fixture:
the pages print no worked LLA values, so the stored numbers are the oracle's own output on
the tiny workload, B1 H1 n64 d16 fp32, seed 0, h = 4, lambda = 1e-2).

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import lla_inputs  # noqa: E402
from oracle import lla_forward  # noqa: E402


def main():
    w = lla_inputs.WORKLOADS["tiny"]
    q, k, v, _ = lla_inputs.generate(w)
    out = lla_forward(q, k, v, w.h, w.lam)[0, 0]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")
    with open(path, "w") as f:
        f.write("# LLA forward, tiny workload (B1 H1 n64 d16 fp32, seed 0, h=4, lambda=1e-2)\n")
        f.write("# written by tests/golden/make_golden.py from oracle/ only; rows i = 0..63\n")
        np.savetxt(f, out, fmt="%.17g")


if __name__ == "__main__":
    main()
