"""ctypes binding of libwhiflash (argument marshalling only).

The shared library is loaded on first use; if it has not been built, the first
call raises WhiflashError.  Nothing here computes any part of the method.
"""

from __future__ import annotations

import ctypes
import os

import torch

WF_F32 = 0
WF_BF16 = 1
WF_OK = 0

_c_p = ctypes.c_void_p
_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_sz = ctypes.c_size_t
_c_f = ctypes.c_float

_SIGNATURES = {
    "whiflash_status_string": (ctypes.c_char_p, [_c_i32]),
    "whiflash_route_workspace_bytes": (_c_sz, [_c_i32, _c_i32]),
    "whiflash_verify_workspace_bytes": (_c_sz, [_c_i32, _c_i32]),
    "whiflash_argmax_sweep_plan": (_c_i32, [_c_i32, _c_i32, _c_p, _c_p]),
    "whiflash_argmax_sweep": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_sz, _c_p]),
    "whiflash_stream_read": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_p]),
    "whiflash_route": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_f,
                                _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_verify_chain": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_p, _c_p,
                                       _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_early_exit_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32]),
    "whiflash_verify_chain_early_exit": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_p,
                                                  _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_tree_early_exit_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32]),
    "whiflash_verify_tree_early_exit": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_p,
                                                 _c_p, _c_p, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                 _c_sz, _c_p]),
    "whiflash_routed_early_exit_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "whiflash_verify_routed_early_exit": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_i32,
                                                   _c_p, _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p,
                                                   _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz,
                                                   _c_p]),
    "whiflash_round_early_exit_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                          _c_i32]),
    "whiflash_round_routed_early_exit": (_c_i32, [_c_p, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p,
                                                  _c_f, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                                  _c_i64, _c_p, _c_i32, _c_i32, _c_p, _c_i32, _c_p,
                                                  _c_p, _c_p, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                  _c_sz, _c_p]),
    "whiflash_verify_routed_entropy_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32]),
    "whiflash_verify_routed_entropy": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_i32,
                                                _c_p, _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p, _c_i32,
                                                _c_f, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                _c_sz, _c_p]),
    "whiflash_round_chain_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "whiflash_round_chain_early_exit_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "whiflash_round_chain_early_exit": (_c_i32, [_c_p, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p,
                                                 _c_p, _c_f, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                                 _c_i32, _c_i32, _c_i64, _c_p, _c_p, _c_p, _c_p,
                                                 _c_p, _c_sz, _c_p]),
    "whiflash_round_chain": (_c_i32, [_c_p, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_f,
                                      _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                      _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_round_chain_noalloc": (_c_i32, [_c_p, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p,
                                              _c_f, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                              _c_i32, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "whiflash_verify_tree": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_p, _c_p,
                                      _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_route_gather": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_i32, _c_p, _c_p,
                                       _c_p, _c_i32, _c_p, _c_p, _c_f, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_round_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "whiflash_round_routed": (_c_i32, [_c_p, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_f,
                                       _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_p,
                                       _c_i32, _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p, _c_i32,
                                       _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_catchup_update": (_c_i32, [_c_i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "whiflash_entropy_workspace_bytes": (_c_sz, [_c_i32, _c_i32]),
    "whiflash_route_entropy": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_p, _c_i32,
                                        _c_p, _c_f, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "whiflash_verify_routed": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_p, _c_i32, _c_p,
                                        _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p, _c_i32, _c_p, _c_p,
                                        _c_p, _c_p, _c_p, _c_sz, _c_p]),
}

_LIB = None


class WhiflashError(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwhiflash.so")


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise WhiflashError(f"{path} is not built: run `python -m drafter_routing_verification_amd.build`")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def status_string(status: int) -> str:
    return lib().whiflash_status_string(status).decode()


def route_workspace_bytes(B: int, m: int) -> int:
    return int(lib().whiflash_route_workspace_bytes(B, m))


def verify_workspace_bytes(total_rows: int, V: int) -> int:
    return int(lib().whiflash_verify_workspace_bytes(total_rows, V))


def argmax_sweep_plan(rows: int, V: int) -> tuple[int, int]:
    """(chunks per row, entries per chunk) of the argmax sweep over rows x V logits."""
    chunks, elems = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().whiflash_argmax_sweep_plan(rows, V, ctypes.byref(chunks), ctypes.byref(elems)))
    return chunks.value, elems.value


# Raw C entry points (integers and pointers), for callers that manage their own memory.
def whiflash_route(*args):
    return lib().whiflash_route(*args)


def whiflash_argmax_sweep(*args):
    return lib().whiflash_argmax_sweep(*args)


def whiflash_stream_read(*args):
    return lib().whiflash_stream_read(*args)


def whiflash_verify_chain(*args):
    return lib().whiflash_verify_chain(*args)


def whiflash_verify_chain_early_exit(*args):
    return lib().whiflash_verify_chain_early_exit(*args)


def early_exit_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(lib().whiflash_early_exit_workspace_bytes(B, K, V))


def whiflash_verify_tree_early_exit(*args):
    return lib().whiflash_verify_tree_early_exit(*args)


def whiflash_verify_routed_early_exit(*args):
    return lib().whiflash_verify_routed_early_exit(*args)


def whiflash_round_routed_early_exit(*args):
    return lib().whiflash_round_routed_early_exit(*args)


def tree_early_exit_workspace_bytes(B: int, N: int, V: int) -> int:
    return int(lib().whiflash_tree_early_exit_workspace_bytes(B, N, V))


def routed_early_exit_workspace_bytes(B: int, K: int, N: int, total_rows: int, V: int) -> int:
    return int(lib().whiflash_routed_early_exit_workspace_bytes(B, K, N, total_rows, V))


def round_early_exit_workspace_bytes(B: int, m: int, K: int, N: int, total_rows: int, V: int) -> int:
    return int(lib().whiflash_round_early_exit_workspace_bytes(B, m, K, N, total_rows, V))


def whiflash_verify_routed_entropy(*args):
    return lib().whiflash_verify_routed_entropy(*args)


def verify_routed_entropy_workspace_bytes(B: int, total_rows: int, V: int) -> int:
    return int(lib().whiflash_verify_routed_entropy_workspace_bytes(B, total_rows, V))


def whiflash_round_chain(*args):
    return lib().whiflash_round_chain(*args)


def whiflash_round_chain_noalloc(*args):
    return lib().whiflash_round_chain_noalloc(*args)


def round_chain_workspace_bytes(B: int, m: int, K: int, V: int) -> int:
    return int(lib().whiflash_round_chain_workspace_bytes(B, m, K, V))


def whiflash_round_chain_early_exit(*args):
    return lib().whiflash_round_chain_early_exit(*args)


def round_chain_early_exit_workspace_bytes(B: int, m: int, K: int, V: int) -> int:
    return int(lib().whiflash_round_chain_early_exit_workspace_bytes(B, m, K, V))


def whiflash_verify_tree(*args):
    return lib().whiflash_verify_tree(*args)


def whiflash_verify_routed(*args):
    return lib().whiflash_verify_routed(*args)


def whiflash_route_gather(*args):
    return lib().whiflash_route_gather(*args)


def whiflash_round_routed(*args):
    return lib().whiflash_round_routed(*args)


def round_workspace_bytes(B: int, m: int, total_rows: int, V: int) -> int:
    return int(lib().whiflash_round_workspace_bytes(B, m, total_rows, V))


def whiflash_catchup_update(*args):
    return lib().whiflash_catchup_update(*args)


def whiflash_route_entropy(*args):
    return lib().whiflash_route_entropy(*args)


def entropy_workspace_bytes(B: int, V: int) -> int:
    return int(lib().whiflash_entropy_workspace_bytes(B, V))


# ----------------------------------------------------------------------------- helpers


def _check(status: int) -> None:
    if status != WF_OK:
        raise WhiflashError(status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return WF_F32
    if t.dtype == torch.bfloat16:
        return WF_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return s.cuda_stream


def _device_tensor(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")


def _i32(t: torch.Tensor, name: str, numel: int | None = None) -> torch.Tensor:
    _device_tensor(t, name)
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, has {t.numel()}")
    return t


def _workspace(ws, nbytes: int, device) -> torch.Tensor | None:
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None
    _device_tensor(ws, "workspace")
    if ws.get_device() != device.index or not ws.is_contiguous():
        raise TypeError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws


def _out(t, dtype: torch.dtype, numel: int, device, name: str) -> torch.Tensor:
    """A caller-supplied output tensor, checked (the kernels write `numel` elements of
    `dtype` through its pointer), or a new one when t is None."""
    if t is None:
        return torch.empty(numel, dtype=dtype, device=device)
    _device_tensor(t, name)
    if t.get_device() != device.index or t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} tensor on {device}")
    if t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} elements, has {t.numel()}")
    return t


def _opt_out(t, numel: int, device, name: str) -> torch.Tensor | None:
    """An optional int32 output: True allocates it, False or None skips it, a tensor is checked."""
    if t is True:
        return torch.empty(max(numel, 1), dtype=torch.int32, device=device)
    if t is False or t is None:
        return None
    return _out(t, torch.int32, numel, device, name)


def _on(device, **tensors) -> None:
    """Every given tensor (None skipped) lives on `device`: the kernels dereference them there."""
    idx = device.index
    for name, t in tensors.items():
        if t is None:
            continue
        _device_tensor(t, name)
        if t.get_device() != idx:
            raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _weights(hidden: torch.Tensor, hidden_name: str, W1, W2) -> None:
    """The hidden states and both router weights: contiguous GPU tensors of one dtype on
    the device of the hidden states."""
    _device_tensor(hidden, hidden_name)
    idx, dt = hidden.get_device(), hidden.dtype
    for t, name in ((hidden, hidden_name), (W1, "W1"), (W2, "W2")):
        _device_tensor(t, name)
        if not t.is_contiguous() or t.dtype != dt:
            raise TypeError(f"{name} must be contiguous with the dtype of {hidden_name}")
        if t.get_device() != idx:
            raise ValueError(f"{name} is on {t.device}, {hidden_name} on {hidden.device}")


def _biases(b1, b2, m: int, device):
    """b1: None or a contiguous float32 tensor of m elements; b2: None, a float, or a
    1-element float32 tensor.  Returns (b1, b2) with b2 as a device tensor or None."""
    if b1 is not None:
        _on(device, b1=b1)
        if b1.dtype != torch.float32 or b1.numel() != m or not b1.is_contiguous():
            raise TypeError("b1 must be a contiguous float32 tensor of m elements")
    if b2 is not None and not isinstance(b2, torch.Tensor):
        b2 = torch.tensor([float(b2)], dtype=torch.float32, device=device)
    if b2 is not None:
        _on(device, b2=b2)
        if b2.dtype != torch.float32 or b2.numel() != 1:
            raise TypeError("b2 must be a float or a 1-element float32 tensor")
    return b1, b2


def _rows_view(logits: torch.Tensor, rows: int) -> tuple[int, int]:
    """(V, row_stride) of a [rows, V] or [B, R, V] logits tensor with unit last stride."""
    _device_tensor(logits, "logits")
    if logits.stride(-1) != 1:
        raise ValueError("logits must have unit stride along the vocabulary")
    V = logits.shape[-1]
    if logits.dim() == 2:
        if logits.shape[0] != rows:
            raise ValueError(f"logits has {logits.shape[0]} rows, expected {rows}")
        if rows > 1:
            return V, logits.stride(0)
        return V, (V + 7) // 8 * 8  # a single row: any aligned stride >= V will do
    if logits.dim() == 3:
        if logits.shape[0] * logits.shape[1] != rows or logits.stride(0) != logits.shape[1] * logits.stride(1):
            raise ValueError("3-D logits must be [B, rows_per_seq, V] with evenly spaced rows")
        return V, logits.stride(1)
    raise ValueError("logits must be 2-D or 3-D")


# ----------------------------------------------------------------------------- entry points


def route(hidden, W1, b1, W2, b2, tau: float, *, delta_al=None, choice=None, workspace=None,
          stream=None):
    """Neural router + threshold.  hidden [B, d], W1 [m, d], W2 [m] (or [1, m]) of one dtype;
    b1 [m] float32 or None; b2 float, 1-element float32 tensor or None."""
    _device_tensor(hidden, "hidden")
    B, d = hidden.shape
    m = W1.shape[0]
    _weights(hidden, "hidden", W1, W2)
    if tuple(W1.shape) != (m, d) or W2.numel() != m:
        raise ValueError("W1 must be [m, d] and W2 hold m elements")
    dev = hidden.device
    b1, b2 = _biases(b1, b2, m, dev)
    delta_al = _out(delta_al, torch.float32, B, dev, "delta_al")
    choice = _out(choice, torch.int32, B, dev, "choice")
    ws = _workspace(workspace, route_workspace_bytes(B, m), dev)
    _check(whiflash_route(_ptr(hidden), _dtype_code(hidden), B, d, _ptr(W1), _ptr(b1), m, _ptr(W2),
                          _ptr(b2), float(tau), _ptr(delta_al), _ptr(choice), _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(hidden, stream)))
    return delta_al, choice


def route_gather(hidden_rows, pos, W1, b1, W2, b2, tau: float, *, row0=None, rows_per_seq: int = 0,
                 delta_al=None, choice=None, workspace=None, stream=None):
    """Neural router on the hidden state at each sequence's final accepted position.
    hidden_rows [total_rows, d]; pos [B] int32; row0 [B] int32 or None with rows_per_seq."""
    _device_tensor(hidden_rows, "hidden_rows")
    _device_tensor(pos, "pos")
    total_rows, d = hidden_rows.shape
    B = pos.numel()
    m = W1.shape[0]
    _weights(hidden_rows, "hidden_rows", W1, W2)
    if tuple(W1.shape) != (m, d) or W2.numel() != m:
        raise ValueError("W1 must be [m, d] and W2 hold m elements")
    _i32(pos, "pos", B)
    if row0 is not None:
        _i32(row0, "row0")
        if row0.numel() < B:
            raise ValueError("row0 must hold at least B entries")
    dev = hidden_rows.device
    b1, b2 = _biases(b1, b2, m, dev)
    delta_al = _out(delta_al, torch.float32, B, dev, "delta_al")
    choice = _out(choice, torch.int32, B, dev, "choice")
    _on(dev, pos=pos, row0=row0)
    ws = _workspace(workspace, route_workspace_bytes(B, m), dev)
    _check(whiflash_route_gather(_ptr(hidden_rows), _dtype_code(hidden_rows), total_rows, d, B,
                                 _ptr(row0), rows_per_seq, _ptr(pos), _ptr(W1), _ptr(b1), m,
                                 _ptr(W2), _ptr(b2), float(tau), _ptr(delta_al), _ptr(choice),
                                 _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                 _stream(hidden_rows, stream)))
    return delta_al, choice


def argmax_sweep(logits, *, rows=None, partials=None, stream=None):
    """The argmax sweep kernel alone over logits [rows, V] (or [B, R, V]).  Returns
    (max float32 [rows, chunks], index int32 [rows, chunks]): each chunk's largest value and
    the lowest row index holding it, chunking from argmax_sweep_plan.  partials: optional
    int32 tensor of at least rows * chunks * 2 elements to write into."""
    if rows is None:
        rows = logits.shape[0] if logits.dim() == 2 else logits.shape[0] * logits.shape[1]
    V, stride = _rows_view(logits, rows)
    chunks, _ = argmax_sweep_plan(rows, V)
    need = rows * chunks * 2
    if partials is None:
        partials = torch.empty(need, dtype=torch.int32, device=logits.device)
    else:
        _i32(partials, "partials")
        _on(logits.device, partials=partials)
        if partials.numel() < need:
            raise ValueError(f"partials needs {need} int32 elements")
    _check(whiflash_argmax_sweep(_ptr(logits), _dtype_code(logits), rows, V, stride,
                                 _ptr(partials), partials.numel() * 4, _stream(logits, stream)))
    rec = partials[:need].view(rows, chunks, 2)
    return rec[..., 0].view(torch.float32), rec[..., 1]


def stream_read(logits, *, rows=None, sink=None, stream=None):
    """Measurement aid: the argmax sweep's reads of logits without its comparisons (same
    chunks, workgroups and loads).  Returns the int32 sink tensor [1] it writes (the XOR of
    the 32-bit words of row 0's first chunk)."""
    if rows is None:
        rows = logits.shape[0] if logits.dim() == 2 else logits.shape[0] * logits.shape[1]
    V, stride = _rows_view(logits, rows)
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=logits.device)
    _i32(sink, "sink")
    _on(logits.device, sink=sink)
    _check(whiflash_stream_read(_ptr(logits), _dtype_code(logits), rows, V, stride, _ptr(sink),
                                _stream(logits, stream)))
    return sink


def verify_chain(logits, draft, *, row_argmax=True, accept_len=None, bonus=None, workspace=None,
                 stream=None):
    """DFlash block verification.  logits [B*(K+1), V] or [B, K+1, V]; draft [B, K] int32.
    row_argmax: True to allocate, a tensor to fill, or False/None to skip."""
    _device_tensor(draft, "draft")
    B, K = draft.shape
    rows = B * (K + 1)
    V, stride = _rows_view(logits, rows)
    _i32(draft, "draft")
    dev = logits.device
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    row_argmax = _opt_out(row_argmax, rows, dev, "row_argmax")
    _on(dev, draft=draft)
    ws = _workspace(workspace, verify_workspace_bytes(rows, V), dev)
    _check(whiflash_verify_chain(_ptr(logits), _dtype_code(logits), B, K, V, stride, _ptr(draft),
                                 _ptr(accept_len), _ptr(bonus), _ptr(row_argmax), _ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(),
                                 _stream(logits, stream)))
    return accept_len, bonus, row_argmax


def verify_chain_early_exit(logits, draft, *, row_argmax=True, accept_len=None, bonus=None,
                            workspace=None, stream=None):
    """DFlash block verification that reads only rows 0..n of each sequence (n = first
    mismatch).  Arguments as verify_chain; row_argmax holds -1 after each sequence's n."""
    _device_tensor(draft, "draft")
    B, K = draft.shape
    rows = B * (K + 1)
    V, stride = _rows_view(logits, rows)
    _i32(draft, "draft")
    dev = logits.device
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    row_argmax = _opt_out(row_argmax, rows, dev, "row_argmax")
    _on(dev, draft=draft)
    ws = _workspace(workspace, early_exit_workspace_bytes(B, K, V), dev)
    _check(whiflash_verify_chain_early_exit(_ptr(logits), _dtype_code(logits), B, K, V, stride,
                                            _ptr(draft), _ptr(accept_len), _ptr(bonus),
                                            _ptr(row_argmax), _ptr(ws),
                                            0 if ws is None else ws.numel() * ws.element_size(),
                                            _stream(logits, stream)))
    return accept_len, bonus, row_argmax


def verify_tree(logits, parent, draft_ids, d2t, *, row_argmax=True, accept_len=None, bonus=None,
                best_node=None, workspace=None, stream=None, _early=False):
    """EAGLE-3 tree verification.  logits [B*N, V] or [B, N, V]; parent, draft_ids [B, N] int32;
    d2t [Vd] int32."""
    _device_tensor(parent, "parent")
    B, N = parent.shape
    rows = B * N
    V, stride = _rows_view(logits, rows)
    _i32(parent, "parent")
    _i32(draft_ids, "draft_ids", B * N)
    _i32(d2t, "d2t")
    dev = logits.device
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    best_node = _out(best_node, torch.int32, B, dev, "best_node")
    row_argmax = _opt_out(row_argmax, rows, dev, "row_argmax")
    _on(dev, parent=parent, draft_ids=draft_ids, d2t=d2t)
    nbytes = tree_early_exit_workspace_bytes(B, N, V) if _early else verify_workspace_bytes(rows, V)
    ws = _workspace(workspace, nbytes, dev)
    fn = whiflash_verify_tree_early_exit if _early else whiflash_verify_tree
    _check(fn(_ptr(logits), _dtype_code(logits), B, N, V, stride, _ptr(parent),
                                _ptr(draft_ids), _ptr(d2t), d2t.numel(), _ptr(accept_len),
                                _ptr(bonus), _ptr(best_node), _ptr(row_argmax), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(logits, stream)))
    return accept_len, bonus, best_node, row_argmax


def verify_routed(logits, row_offsets, total_rows: int, choice, chain_draft, parent, draft_ids, d2t,
                  *, row_argmax=True, accept_len=None, bonus=None, best_node=None, workspace=None,
                  stream=None, _early=False):
    """Routed ragged batch.  logits [total_rows, V] packed; row_offsets [B+1], choice [B],
    chain_draft [B, K], parent and draft_ids [B, N], d2t [Vd] -- all int32 device tensors."""
    _device_tensor(choice, "choice")
    B = choice.numel()
    if logits.dim() != 2:
        raise ValueError("routed logits must be [total_rows, V]")
    V, stride = _rows_view(logits, total_rows)
    _i32(row_offsets, "row_offsets", B + 1)
    _i32(choice, "choice", B)
    K = chain_draft.shape[1]
    N = parent.shape[1]
    _i32(chain_draft, "chain_draft", B * K)
    _i32(parent, "parent", B * N)
    _i32(draft_ids, "draft_ids", B * N)
    _i32(d2t, "d2t")
    dev = logits.device
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    best_node = _out(best_node, torch.int32, B, dev, "best_node")
    row_argmax = _opt_out(row_argmax, total_rows, dev, "row_argmax")
    _on(dev, row_offsets=row_offsets, choice=choice, chain_draft=chain_draft, parent=parent,
        draft_ids=draft_ids, d2t=d2t)
    nbytes = (routed_early_exit_workspace_bytes(B, K, N, total_rows, V) if _early
              else verify_workspace_bytes(total_rows, V))
    ws = _workspace(workspace, nbytes, dev)
    fn = whiflash_verify_routed_early_exit if _early else whiflash_verify_routed
    _check(fn(_ptr(logits), _dtype_code(logits), B, V, stride, _ptr(row_offsets),
                                  total_rows, _ptr(choice), K, _ptr(chain_draft), N, _ptr(parent),
                                  _ptr(draft_ids), _ptr(d2t), d2t.numel(), _ptr(accept_len),
                                  _ptr(bonus), _ptr(best_node), _ptr(row_argmax), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(logits, stream)))
    return accept_len, bonus, best_node, row_argmax


def route_entropy(logits, pos, tau: float, *, row0=None, rows_per_seq: int = 0, entropy=None,
                  choice=None, workspace=None, stream=None):
    """WhiFlash-Entropy policy.  logits [total_rows, V] (or [B, R, V]); pos [B] int32 position of
    each sequence's final accepted row within the sequence; row0 [B] int32 first row of each
    sequence, or None with rows_per_seq (row0[b] = b * rows_per_seq)."""
    _device_tensor(pos, "pos")
    B = pos.numel()
    if logits.dim() == 3:
        total_rows = logits.shape[0] * logits.shape[1]
    else:
        total_rows = logits.shape[0]
    V, stride = _rows_view(logits, total_rows)
    _i32(pos, "pos", B)
    if row0 is not None:
        _i32(row0, "row0")
        if row0.numel() < B:
            raise ValueError("row0 must hold at least B entries")
    dev = logits.device
    entropy = _out(entropy, torch.float32, B, dev, "entropy")
    choice = _out(choice, torch.int32, B, dev, "choice")
    _on(dev, pos=pos, row0=row0)
    ws = _workspace(workspace, entropy_workspace_bytes(B, V), dev)
    _check(whiflash_route_entropy(_ptr(logits), _dtype_code(logits), total_rows, V, stride, B,
                                  _ptr(row0), rows_per_seq, _ptr(pos), float(tau), _ptr(entropy),
                                  _ptr(choice), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(logits, stream)))
    return entropy, choice


def catchup_update(cur_choice, accept_len, next_choice, backlog, *, switch_flag=True,
                   catchup_len=True, stream=None):
    """Lazy catch-up bookkeeping; backlog [B, 2] int32 is updated in place.
    Returns (switch_flag, catchup_len) (None where not requested)."""
    B = cur_choice.numel()
    _i32(cur_choice, "cur_choice", B)
    _i32(accept_len, "accept_len", B)
    _i32(next_choice, "next_choice", B)
    _i32(backlog, "backlog", 2 * B)
    dev = backlog.device
    switch_flag = _opt_out(switch_flag, B, dev, "switch_flag")
    catchup_len = _opt_out(catchup_len, B, dev, "catchup_len")
    _on(dev, cur_choice=cur_choice, accept_len=accept_len, next_choice=next_choice)
    _check(whiflash_catchup_update(B, _ptr(cur_choice), _ptr(accept_len), _ptr(next_choice),
                                   _ptr(backlog), _ptr(switch_flag), _ptr(catchup_len),
                                   _stream(backlog, stream)))
    return switch_flag, catchup_len


def round_routed(hidden, W1, b1, W2, b2, tau: float, logits, row_offsets, total_rows: int,
                 chain_draft, parent, draft_ids, d2t, *, row_argmax=True, delta_al=None,
                 choice=None, accept_len=None, bonus=None, best_node=None, workspace=None,
                 stream=None, _early=False):
    """route + verify_routed in one call (three launches; two when the router is small enough
    to share the sweep's launch).  Returns (delta_al, choice, accept_len, bonus, best_node,
    row_argmax)."""
    _device_tensor(hidden, "hidden")
    B, d = hidden.shape
    m = W1.shape[0]
    _weights(hidden, "hidden", W1, W2)
    if tuple(W1.shape) != (m, d) or W2.numel() != m:
        raise ValueError("W1 must be [m, d] and W2 hold m elements")
    dev = hidden.device
    b1, b2 = _biases(b1, b2, m, dev)
    if logits.dim() != 2:
        raise ValueError("routed logits must be [total_rows, V]")
    V, stride = _rows_view(logits, total_rows)
    _i32(row_offsets, "row_offsets", B + 1)
    K = chain_draft.shape[1]
    N = parent.shape[1]
    _i32(chain_draft, "chain_draft", B * K)
    _i32(parent, "parent", B * N)
    _i32(draft_ids, "draft_ids", B * N)
    _i32(d2t, "d2t")
    delta_al = _out(delta_al, torch.float32, B, dev, "delta_al")
    choice = _out(choice, torch.int32, B, dev, "choice")
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    best_node = _out(best_node, torch.int32, B, dev, "best_node")
    row_argmax = _opt_out(row_argmax, total_rows, dev, "row_argmax")
    _on(dev, logits=logits, row_offsets=row_offsets, chain_draft=chain_draft, parent=parent,
        draft_ids=draft_ids, d2t=d2t)
    nbytes = (round_early_exit_workspace_bytes(B, m, K, N, total_rows, V) if _early
              else round_workspace_bytes(B, m, total_rows, V))
    ws = _workspace(workspace, nbytes, dev)
    fn = whiflash_round_routed_early_exit if _early else whiflash_round_routed
    _check(fn(_ptr(hidden), _dtype_code(hidden), d, _ptr(W1), _ptr(b1), m,
                                 _ptr(W2), _ptr(b2), float(tau), _ptr(delta_al), _ptr(choice),
                                 _ptr(logits), _dtype_code(logits), B, V, stride, _ptr(row_offsets),
                                 total_rows, K, _ptr(chain_draft), N, _ptr(parent), _ptr(draft_ids),
                                 _ptr(d2t), d2t.numel(), _ptr(accept_len), _ptr(bonus),
                                 _ptr(best_node), _ptr(row_argmax), _ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(),
                                 _stream(hidden, stream)))
    return delta_al, choice, accept_len, bonus, best_node, row_argmax


def verify_tree_early_exit(logits, parent, draft_ids, d2t, **kw):
    """verify_tree that reads only the rows of accepted nodes (row_argmax -1 elsewhere)."""
    return verify_tree(logits, parent, draft_ids, d2t, _early=True, **kw)


def verify_routed_early_exit(logits, row_offsets, total_rows: int, choice, chain_draft, parent,
                             draft_ids, d2t, **kw):
    """verify_routed that reads only the rows of accepted nodes (row_argmax -1 elsewhere)."""
    return verify_routed(logits, row_offsets, total_rows, choice, chain_draft, parent, draft_ids, d2t,
                         _early=True, **kw)


def round_routed_early_exit(hidden, W1, b1, W2, b2, tau: float, logits, row_offsets, total_rows: int,
                            chain_draft, parent, draft_ids, d2t, **kw):
    """round_routed with the early-exit verification (four launches)."""
    return round_routed(hidden, W1, b1, W2, b2, tau, logits, row_offsets, total_rows, chain_draft,
                        parent, draft_ids, d2t, _early=True, **kw)


def verify_routed_entropy(logits, row_offsets, total_rows: int, choice, chain_draft, parent,
                          draft_ids, d2t, tau: float, *, row_argmax=True, accept_len=None,
                          bonus=None, best_node=None, entropy=None, next_choice=None,
                          workspace=None, stream=None):
    """verify_routed plus the entropy policy at each accepted row (one call).
    Returns (accept_len, bonus, best_node, row_argmax, entropy, next_choice)."""
    _device_tensor(choice, "choice")
    B = choice.numel()
    if logits.dim() != 2:
        raise ValueError("routed logits must be [total_rows, V]")
    V, stride = _rows_view(logits, total_rows)
    _i32(row_offsets, "row_offsets", B + 1)
    _i32(choice, "choice", B)
    K = chain_draft.shape[1]
    N = parent.shape[1]
    _i32(chain_draft, "chain_draft", B * K)
    _i32(parent, "parent", B * N)
    _i32(draft_ids, "draft_ids", B * N)
    _i32(d2t, "d2t")
    dev = logits.device
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    best_node = _out(best_node, torch.int32, B, dev, "best_node")
    entropy = _out(entropy, torch.float32, B, dev, "entropy")
    next_choice = _out(next_choice, torch.int32, B, dev, "next_choice")
    row_argmax = _opt_out(row_argmax, total_rows, dev, "row_argmax")
    _on(dev, row_offsets=row_offsets, choice=choice, chain_draft=chain_draft, parent=parent,
        draft_ids=draft_ids, d2t=d2t)
    ws = _workspace(workspace, verify_routed_entropy_workspace_bytes(B, total_rows, V), dev)
    _check(whiflash_verify_routed_entropy(
        _ptr(logits), _dtype_code(logits), B, V, stride, _ptr(row_offsets), total_rows,
        _ptr(choice), K, _ptr(chain_draft), N, _ptr(parent), _ptr(draft_ids), _ptr(d2t),
        d2t.numel(), float(tau), _ptr(accept_len), _ptr(bonus), _ptr(best_node), _ptr(row_argmax),
        _ptr(entropy), _ptr(next_choice), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(logits, stream)))
    return accept_len, bonus, best_node, row_argmax, entropy, next_choice


def round_chain(hidden, W1, b1, W2, b2, tau: float, logits, draft, *, row_argmax=True,
                delta_al=None, choice=None, accept_len=None, bonus=None, workspace=None,
                stream=None, _early=False):
    """route + verify_chain in one call (three launches; two when the router is small enough
    to share the sweep's launch).  hidden [B, d]; logits [B*(K+1), V] or [B, K+1, V]; draft
    [B, K] int32.  Returns (delta_al, choice, accept_len, bonus, row_argmax)."""
    _device_tensor(hidden, "hidden")
    B, d = hidden.shape
    m = W1.shape[0]
    _weights(hidden, "hidden", W1, W2)
    if tuple(W1.shape) != (m, d) or W2.numel() != m:
        raise ValueError("W1 must be [m, d] and W2 hold m elements")
    dev = hidden.device
    b1, b2 = _biases(b1, b2, m, dev)
    _device_tensor(draft, "draft")
    if draft.shape[0] != B:
        raise ValueError("draft must be [B, K] with the batch of hidden")
    K = draft.shape[1]
    rows = B * (K + 1)
    V, stride = _rows_view(logits, rows)
    _i32(draft, "draft")
    delta_al = _out(delta_al, torch.float32, B, dev, "delta_al")
    choice = _out(choice, torch.int32, B, dev, "choice")
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    row_argmax = _opt_out(row_argmax, rows, dev, "row_argmax")
    _on(dev, logits=logits, draft=draft)
    nbytes = (round_chain_early_exit_workspace_bytes(B, m, K, V) if _early
              else round_chain_workspace_bytes(B, m, K, V))
    ws = _workspace(workspace, nbytes, dev)
    fn = whiflash_round_chain_early_exit if _early else whiflash_round_chain
    _check(fn(_ptr(hidden), _dtype_code(hidden), d, _ptr(W1), _ptr(b1), m,
                                _ptr(W2), _ptr(b2), float(tau), _ptr(delta_al), _ptr(choice),
                                _ptr(logits), _dtype_code(logits), B, K, V, stride, _ptr(draft),
                                _ptr(accept_len), _ptr(bonus), _ptr(row_argmax), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(hidden, stream)))
    return delta_al, choice, accept_len, bonus, row_argmax


def round_chain_noalloc(hidden, W1, b1, W2, b2, tau: float, logits, draft, *, row_argmax=True,
                        delta_al=None, choice=None, accept_len=None, bonus=None, stream=None):
    """round_chain with the library's fixed device scratch instead of a workspace
    (whiflash_round_chain_noalloc: the C call allocates nothing; outputs the caller does not
    supply are allocated here).  Calls that overlap in time on one GPU race on the scratch."""
    _device_tensor(hidden, "hidden")
    B, d = hidden.shape
    m = W1.shape[0]
    _weights(hidden, "hidden", W1, W2)
    if tuple(W1.shape) != (m, d) or W2.numel() != m:
        raise ValueError("W1 must be [m, d] and W2 hold m elements")
    dev = hidden.device
    b1, b2 = _biases(b1, b2, m, dev)
    _device_tensor(draft, "draft")
    if draft.shape[0] != B:
        raise ValueError("draft must be [B, K] with the batch of hidden")
    K = draft.shape[1]
    rows = B * (K + 1)
    V, stride = _rows_view(logits, rows)
    _i32(draft, "draft")
    delta_al = _out(delta_al, torch.float32, B, dev, "delta_al")
    choice = _out(choice, torch.int32, B, dev, "choice")
    accept_len = _out(accept_len, torch.int32, B, dev, "accept_len")
    bonus = _out(bonus, torch.int32, B, dev, "bonus")
    row_argmax = _opt_out(row_argmax, rows, dev, "row_argmax")
    _on(dev, logits=logits, draft=draft)
    _check(whiflash_round_chain_noalloc(
        _ptr(hidden), _dtype_code(hidden), d, _ptr(W1), _ptr(b1), m, _ptr(W2), _ptr(b2),
        float(tau), _ptr(delta_al), _ptr(choice), _ptr(logits), _dtype_code(logits), B, K, V,
        stride, _ptr(draft), _ptr(accept_len), _ptr(bonus), _ptr(row_argmax),
        _stream(hidden, stream)))
    return delta_al, choice, accept_len, bonus, row_argmax


def round_chain_early_exit(hidden, W1, b1, W2, b2, tau: float, logits, draft, **kw):
    """round_chain with the early-exit verification (row_argmax -1 after each first mismatch)."""
    return round_chain(hidden, W1, b1, W2, b2, tau, logits, draft, _early=True, **kw)
