import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _have_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _have_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """The largest Delta-AL error the router comparisons saw, per input element type."""
    mod = sys.modules.get("gpu_helpers")
    seen = getattr(mod, "OBSERVED_DAL_ERR", None) if mod else None
    if seen:
        for dtype, (err, batch) in sorted(seen.items()):
            terminalreporter.write_line(
                f"largest delta-AL error, {dtype} inputs: {err:.3e} relative "
                f"(tolerance rule |gpu - ref| <= rtol * max(|ref|, 1); batch {batch})")
