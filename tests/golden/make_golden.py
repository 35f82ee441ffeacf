"""Writes tiny_oracle.txt: the oracle's outputs on the tiny workload (seed 0).

Calls only ``oracle/`` and the seeded input generator.  The file is a
regression snapshot of the oracle's arithmetic: any later change to that
arithmetic shows up as a diff of this file.
Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from gdn_inputs import WORKLOADS, make_inputs  # noqa: E402
from oracle import gdn_oracle as O  # noqa: E402


def main():
    w = WORKLOADS[0]
    x = make_inputs(w, 0)
    a = (x["q"], x["k"], x["v"], x["log_gate"], x["beta"])
    lines = [f"# oracle outputs, workload {w.name}, seed 0; rows are tokens, columns d_v"]
    for mode in ("fwd", "bwd", "bidir"):
        o, H = O.forward(mode, *a, x["h0"])
        lines.append(f"[{mode}.out] {o.shape[1]}x{o.shape[3]}")
        lines += [" ".join(f"{val:.17g}" for val in row) for row in o[0, :, 0]]
        lines.append(f"[{mode}.state] {H.shape[2]}x{H.shape[3]}")
        lines += [" ".join(f"{val:.17g}" for val in row) for row in H[0, 0]]
    with open(os.path.join(HERE, "tiny_oracle.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
