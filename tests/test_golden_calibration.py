"""The routed workload's stored calibration is reproducible from the committed tree.

tests/golden/routed_calibration.json (b2 and the 64/64 drafter layout of the
routed mixed batch) is written by tests/golden/make_routed_calibration.py, which
calls only the oracle and the seeded generators.  This reruns that writer into a
temporary directory and compares the result with the stored file byte for byte.
"""

import filecmp
import importlib.util
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _writer():
    spec = importlib.util.spec_from_file_location(
        "make_routed_calibration", os.path.join(GOLDEN, "make_routed_calibration.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_routed_calibration_regenerates_byte_for_byte(tmp_path):
    out = tmp_path / "routed_calibration.json"
    _writer().write(str(out))
    assert filecmp.cmp(out, os.path.join(GOLDEN, "routed_calibration.json"), shallow=False)


def test_routed_calibration_is_an_exact_split_with_margin():
    with open(os.path.join(GOLDEN, "routed_calibration.json")) as f:
        cal = json.load(f)
    choice = np.asarray(cal["choice"])
    assert choice.shape == (128,) and set(choice.tolist()) <= {0, 1}
    assert int(choice.sum()) == 64
    assert cal["min_margin"] >= 1e-3
