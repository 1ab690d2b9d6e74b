"""Writes the stored expected values under tests/golden/ (calls only oracle/).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle.cca as O  # noqa: E402
from synth import CCAShape, make_prefill  # noqa: E402


def tiny_prefill():
    s = CCAShape(batch=1, seq_len=5, d_model=8, n_q_heads=2, n_kv_heads=2, head_dim=4,
                 rope_base=100.0, dtype="f32")
    P = make_prefill(s, 0)
    y = O.prefill(P.x, P.weights.f64(), s)
    return {
        "source": "oracle.cca.prefill on synth.make_prefill(shape, seed=0); regression pin of "
                  "the oracle itself, not a value printed by the pages",
        "shape": s.as_dict(),
        "y": [[[float(v) for v in row] for row in yb] for yb in y],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_prefill_oracle.json"), "w") as f:
        json.dump(tiny_prefill(), f, indent=1)
    print("wrote tiny_prefill_oracle.json")
