"""Writes routed_calibration.json: the second-layer bias b2 and the per-sequence
drafter choices of the routed mixed-batch workload (128 sequences, bf16 hidden
states, router 2560 -> 1024 -> 1, threshold 1.0).

Calls only the oracle and the seeded generators.  b2 is set so that the
threshold falls midway between the 64th and 65th predicted gains, giving an
exact 64/64 split with every sequence at least 1e-3 away from the threshold.

    python tests/golden/make_routed_calibration.py [OUTPUT_PATH]

With no argument it rewrites the stored file next to this script.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import route                                      # noqa: E402
from synth.workloads import CONFIGS, TAU, make_router_inputs  # noqa: E402

WORKLOAD = "routed_bf16"
STORED = os.path.join(HERE, "routed_calibration.json")


def calibration() -> dict:
    cfg = CONFIGS[WORKLOAD]
    r = make_router_inputs(cfg["seed"], cfg["B"], dtype=cfg["dtype"], b2=0.0)
    dal0, _ = route(r.hidden, r.W1, r.b1, r.W2, 0.0, TAU, cfg["dtype"])
    s = np.sort(dal0)
    half = cfg["B"] // 2
    b2 = float(np.float32(TAU - 0.5 * (s[half - 1] + s[half])))
    dal, choice = route(r.hidden, r.W1, r.b1, r.W2, b2, TAU, cfg["dtype"])
    margin = float(np.min(np.abs(dal - TAU)))
    assert int(choice.sum()) == half, choice.sum()
    assert margin >= 1e-3, margin
    return {
        "workload": WORKLOAD,
        "seed": cfg["seed"],
        "tau": TAU,
        "b2": b2,
        "min_margin": margin,
        "choice": [int(c) for c in choice],
        "writer": "tests/golden/make_routed_calibration.py (oracle.route, float64)",
    }


def write(path: str) -> dict:
    out = calibration()
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


if __name__ == "__main__":
    out = write(sys.argv[1] if len(sys.argv) > 1 else STORED)
    print(json.dumps({k: v for k, v in out.items() if k != "choice"}))
