"""The oracle still reproduces its committed snapshot on the tiny workload (CPU)."""
import os

import numpy as np

from gdn_inputs import WORKLOADS, make_inputs
from oracle import gdn_oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden():
    out, cur = {}, None
    for line in open(os.path.join(HERE, "tiny_oracle.txt")):
        if line.startswith("#"):
            continue
        if line.startswith("["):
            cur = line[1:line.index("]")]
            out[cur] = []
        else:
            out[cur].append([float(t) for t in line.split()])
    return {k: np.array(v) for k, v in out.items()}


def test_oracle_reproduces_snapshot():
    g = load_golden()
    x = make_inputs(WORKLOADS[0], 0)
    a = (x["q"], x["k"], x["v"], x["log_gate"], x["beta"])
    for mode in ("fwd", "bwd", "bidir"):
        o, H = O.forward(mode, *a, x["h0"])
        np.testing.assert_allclose(o[0, :, 0], g[f"{mode}.out"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(H[0, 0], g[f"{mode}.state"], rtol=0, atol=1e-13)
