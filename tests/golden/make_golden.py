"""Writes oracle_tiny.json: small regression fixtures produced by the oracle alone.

The pages print no numeric worked example for the TTT scan, so these fixtures are
not an external pin: they freeze the oracle's present output on a few tiny,
hand-picked inputs (ragged last chunk, per-token eta, MLP with and without
biases) so that any later change to its arithmetic shows up in review.  Run from
the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(2024)
    cases = []
    d, T = 3, 7
    K = np.round(rng.standard_normal((1, T, d)), 3)
    Q = np.round(rng.standard_normal((1, T, d)), 3)
    V = np.round(rng.standard_normal((1, T, d)), 3)
    eta = np.round(rng.uniform(0.05, 0.3, (1, T)), 3)
    W0 = np.round(rng.standard_normal((1, d, d)) * 0.5, 3)
    for chunk, e in ((3, eta), (2, None), (1, eta)):
        Z, W = oracle.linear(K, Q, V, e, 0.25, W0, chunk=chunk)
        cases.append({"model": "linear", "chunk": chunk, "eta_scalar": 0.25,
                      "inputs": {"K": K.tolist(), "Q": Q.tolist(), "V": V.tolist(),
                                 "eta": None if e is None else e.tolist(), "W0": W0.tolist()},
                      "outputs": {"Z": Z.tolist(), "W": W.tolist()}})
    hd = 4
    W1 = np.round(rng.standard_normal((1, hd, d)) * 0.5, 3)
    b1 = np.round(rng.standard_normal((1, hd)) * 0.2, 3)
    W2 = np.round(rng.standard_normal((1, d, hd)) * 0.5, 3)
    b2 = np.round(rng.standard_normal((1, d)) * 0.2, 3)
    for chunk, bias in ((3, True), (4, False)):
        o = oracle.mlp(K, Q, V, eta, 0.0, W1, b1 if bias else None, W2, b2 if bias else None,
                       chunk=chunk)
        outs = {"Z": o[0].tolist(), "W1": o[1].tolist(), "W2": o[3].tolist()}
        if bias:
            outs["b1"] = o[2].tolist()
            outs["b2"] = o[4].tolist()
        cases.append({"model": "mlp", "chunk": chunk, "eta_scalar": 0.0,
                      "inputs": {"K": K.tolist(), "Q": Q.tolist(), "V": V.tolist(),
                                 "eta": eta.tolist(), "W1": W1.tolist(),
                                 "b1": b1.tolist() if bias else None, "W2": W2.tolist(),
                                 "b2": b2.tolist() if bias else None},
                      "outputs": outs})
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(out, "w") as f:
        json.dump({"note": "written by tests/golden/make_golden.py from the oracle only",
                   "cases": cases}, f, indent=1)


if __name__ == "__main__":
    main()
