"""Writes tests/golden/fc_oracle.json from the oracle alone (fc workload: a[32x64],
g[32x16] fp32 N(0,1) from seed 1, dW = g^T a / 32, no bias column, damping
sqrt(1e-3) per factor). Run from the repository root: python tests/golden/make_fc_golden.py"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402
import synth   # noqa: E402


def main():
    seed = synth.config_seed("fc")
    a = synth.normal_f32(synth.layer_rng(seed, 0), (32, 64))
    g = synth.normal_f32(synth.layer_rng(seed, 1), (32, 16))
    dW = (g.astype(np.float64).T @ a.astype(np.float64)) / 32.0
    s = float(np.float32(np.sqrt(1e-3)))
    A, G = oracle.conv_factors(a.reshape(32, 1, 1, 64), g.reshape(32, 1, 1, 16),
                               1, 1, 1, 1, 0, 0, 0)
    Ai, _ = oracle.damped_inverse(A, s)
    Gi, _ = oracle.damped_inverse(G, s)
    P = oracle.precondition(Gi, dW, Ai)
    out = {"_source": "written by tests/golden/make_fc_golden.py from oracle/ only"}
    rng = np.random.default_rng(0)
    for name, v in (("A", A), ("G", G), ("A_inv", Ai), ("G_inv", Gi), ("P", P)):
        idx = [[int(rng.integers(v.shape[0])), int(rng.integers(v.shape[1]))] for _ in range(6)]
        out[name] = {"fro": float(np.linalg.norm(v)), "idx": idx,
                     "val": [float(v[i, j]) for i, j in idx]}
    with open(os.path.join(ROOT, "tests", "golden", "fc_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
