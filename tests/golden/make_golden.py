"""Write tests/golden/csa_small.json: a small fixed case evaluated by the oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import csa_reference  # noqa: E402


def main():
    # hand-written decimal inputs: B = H = 1, T = 5, d = 2, d_v = 3, non-zero k_0, v_0
    q = [[[[0.5, -1.0], [1.25, 0.75], [-0.5, 2.0], [0.0, 0.0], [3.0, -2.5]]]]
    k = [[[[1.0, 0.5], [-0.25, 1.5], [2.0, -1.0], [0.75, 0.25], [-1.5, -0.5]]]]
    v = [[[[1.0, 0.0, -1.0], [0.5, 2.0, 0.25], [-1.0, 1.0, 3.0], [2.0, -0.5, 0.0], [0.0, 1.5, -2.0]]]]
    k0 = [[[0.25, -0.75]]]
    v0 = [[[-0.5, 0.5, 1.0]]]
    o, lse = csa_reference(np.array(q), np.array(k), np.array(v), np.array(k0), np.array(v0))
    out = {
        "source": "oracle.csa_reference (eq. (8) of J. Su, Continuous Softmax Attention); "
                  "written by tests/golden/make_golden.py",
        "q": q, "k": k, "v": v, "k0": k0, "v0": v0,
        "o": o.tolist(), "lse": lse.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csa_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
