"""Write tests/golden/tiny_512x256.json: digests of the CPU oracle's outputs on
the tiny BitLinear workload (W fp32 512 x 256 ~ N(0, 0.02^2), X fp32 16 x 256 ~
N(0, 1)).  Calls only the oracle and the seeded generators.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import synth, workloads  # noqa: E402


def digest(a):
    return hashlib.sha256(a.tobytes()).hexdigest()


def tiny_outputs():
    wl = workloads.TINY
    layer = wl.layers[0]
    w = synth.latent_weights(layer.N, layer.K, seed=workloads.seed_for(wl, 0, 0))
    x = synth.activations_f32(wl.batches[0], layer.K, seed=workloads.seed_for(wl, 0, 1))
    t, g = oracle.quantize_weights(w)
    out = oracle.forward(t, g, x)
    return {
        "gamma_bits": int(g.view("<u4")),
        "T": digest(t),
        "P_i2": digest(oracle.pack(t, oracle.LAYOUT_I2)),
        "P_b3": digest(oracle.pack(t, oracle.LAYOUT_B3)),
        "q": digest(out["q"]),
        "beta": digest(out["beta"]),
        "acc": digest(out["acc"]),
        "y": digest(out["y"]),
        "zero_fraction": float((t == 0).mean()),
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_512x256.json")
    with open(path, "w") as f:
        json.dump({"_about": "written by tests/golden/make_golden.py from the CPU oracle only",
                   **tiny_outputs()}, f, indent=1)
        f.write("\n")
    print("wrote", path)
