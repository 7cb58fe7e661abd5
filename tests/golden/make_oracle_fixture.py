"""Writes oracle_tiny_fixture.json: the fp64 oracle's outputs on a tiny seeded
case (both NLL scopes).  Calls only the oracle; inputs are drawn here with a
plain NumPy generator.  Run from the repository root:
    python tests/golden/make_oracle_fixture.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import cce_oracle as O  # noqa: E402


def main():
    rng = np.random.default_rng(20261202)
    # two pairs: pair 0 = 2 prompt, 3 chosen, 2 rejected, 1 ignore; pair 1 = 0, 2, 3
    kinds = [1, 1, 2, 2, 2, 3, 3, 0] + [2, 2, 3, 3, 3]
    pairs = [0] * 8 + [1] * 5
    seg = [(p << 2) | k for p, k in zip(pairs, kinds)]
    M, D, V = len(seg), 5, 9
    H = np.round(rng.standard_normal((M, D)) * 1.5, 3)
    W = np.round(rng.standard_normal((V, D)) * 0.7, 3)
    y = rng.integers(0, V, size=M)
    y[np.array(kinds) == 0] = -1
    fx = dict(H=H.tolist(), W=W.tolist(), y=y.tolist(), seg=seg, n_pairs=2, **{"lambda": 0.3})
    for sc, key in ((O.SCOPE_FULL, "full"), (O.SCOPE_RESPONSE, "response")):
        out = O.step(H, W, y, np.array(seg), 2, 0.3, sc)
        fx[key] = {k: (out[k].tolist() if isinstance(out[k], np.ndarray) else float(out[k]))
                   for k in ("loss", "nll", "orv", "margin", "accuracy", "logp", "lse", "coef", "dh", "dW")}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_fixture.json")
    with open(path, "w") as f:
        json.dump(fx, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
