"""Writes routed_calibration.json: the second-layer bias b2 and the per-sequence
drafter choices of the routed mixed-batch workload (128 sequences, bf16 hidden
states, router 2560 -> 1024 -> 1, threshold 1.0).

Calls only the oracle and the seeded generators.  b2 is set so that the
threshold falls midway between the 64th and 65th predicted gains, giving an
exact 64/64 split with every sequence at least `margin` away from the threshold.

    python tests/golden/make_routed_calibration.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import route                       # noqa: E402
from synth.workloads import CONFIGS, TAU, make_router_inputs  # noqa: E402

cfg = CONFIGS["routed_bf16"]
r = make_router_inputs(cfg["seed"], cfg["B"], dtype=cfg["dtype"], b2=0.0)
dal0, _ = route(r.hidden, r.W1, r.b1, r.W2, 0.0, TAU, cfg["dtype"])
s = np.sort(dal0)
half = cfg["B"] // 2
b2 = float(np.float32(TAU - 0.5 * (s[half - 1] + s[half])))
dal, choice = route(r.hidden, r.W1, r.b1, r.W2, b2, TAU, cfg["dtype"])
margin = float(np.min(np.abs(dal - TAU)))
assert int(choice.sum()) == half, choice.sum()
assert margin >= 1e-3, margin
out = {
    "workload": cfg["name"],
    "seed": cfg["seed"],
    "tau": TAU,
    "b2": b2,
    "min_margin": margin,
    "choice": [int(c) for c in choice],
    "writer": "tests/golden/make_routed_calibration.py (oracle.route, float64)",
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "routed_calibration.json"), "w") as f:
    json.dump(out, f, indent=1)
print(json.dumps({k: v for k, v in out.items() if k != "choice"}))
