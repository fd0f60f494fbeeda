"""Write the oracle regression fixture (calls only oracle/ and synth/).

The pages print no worked numeric example of the layer, so the only stored
expected values are these: float64 oracle outputs on a tiny seeded input,
kept so an accidental change to the oracle's arithmetic shows up. Run from
the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import prefill_inputs  # noqa: E402

inputs = dict(B=1, T=70, H_q=4, H_kv=2, d=8, dtype="bf16", seed=123)
x = prefill_inputs(**inputs)
o, S = oracle.prefill(x["q"], x["k"], x["v"], oracle.VECTOR_AVGPOOL4, 16, 0.5)
rng = np.random.default_rng(0)
o_idx = np.sort(rng.choice(o.size, 64, replace=False))
S_idx = np.sort(rng.choice(S.size, 32, replace=False))
fx = dict(
    note="float64 oracle outputs; written by tests/golden/make_golden.py",
    inputs=inputs, gate_mode=oracle.VECTOR_AVGPOOL4, window=16, alpha=0.5,
    o_index=o_idx.tolist(), o_values=[float(a) for a in o.ravel()[o_idx]],
    S_index=S_idx.tolist(), S_values=[float(a) for a in S.ravel()[S_idx]],
)
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_prefill_small.json"), "w") as f:
    json.dump(fx, f, indent=1)
print("wrote oracle_prefill_small.json")
