"""Shared helpers of the GPU parity tests: host arrays to device tensors, padded
logits storage, and the tolerance rules of the router comparison."""

import numpy as np
import torch

DEV = "cuda:0"

# Delta-AL tolerance: |gpu - ref| <= rtol * max(|ref|, 1).  Choices must match
# except where the exact gain lies within NEAR of the threshold.
RTOL = {"f32": 1e-4, "bf16": 2e-2}
NEAR = 1e-3


def dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """Host array -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 or dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def padded_logits(raw: np.ndarray, stride: int) -> torch.Tensor:
    """[rows, V] logits stored with a row stride of `stride` elements (padding filled with +inf
    bit patterns, so reading past V would change the argmax)."""
    rows, V = raw.shape
    if raw.dtype == np.uint16:
        buf = np.full((rows, stride), 0x7F80, np.uint16)
    else:
        buf = np.full((rows, stride), np.inf, np.float32)
    buf[:, :V] = raw
    return dev(buf)[:, :V]


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


# Largest Delta-AL error seen per input element type in this session, with the
# router shape it came from; printed at the end of the run (conftest.py).
OBSERVED_DAL_ERR: dict = {}


def check_router(dal_gpu, ch_gpu, dal_ref, ch_ref, dtype, tau):
    dal_gpu = np.asarray(dal_gpu, np.float64)
    err = np.abs(dal_gpu - dal_ref) / np.maximum(np.abs(dal_ref), 1.0)
    assert err.max() <= RTOL[dtype], f"delta-AL rel err {err.max():.3e} > {RTOL[dtype]}"
    far = np.abs(dal_ref - tau) >= NEAR
    assert np.array_equal(np.asarray(ch_gpu)[far], ch_ref[far]), "routing choices differ"
    worst = float(err.max()) if err.size else 0.0
    if worst >= OBSERVED_DAL_ERR.get(dtype, (-1.0, 0))[0]:
        OBSERVED_DAL_ERR[dtype] = (worst, len(dal_gpu))
    return worst
