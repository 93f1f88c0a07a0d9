"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol the header declares, sizes workspaces, and rejects bad arguments with the
documented status codes before launching anything."""

import os
import re

import pytest

import drafter_routing_verification_amd as wf

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "whiflash.h")
V = 151936


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(whiflash_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert {"whiflash_route", "whiflash_verify_chain", "whiflash_verify_tree",
            "whiflash_verify_routed"} <= set(names)
    lib = wf.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(-8, 1):
        s = wf.status_string(code)
        assert s.startswith("WF_") and s != "unknown whiflash status"
    assert wf.status_string(5) == "unknown whiflash status"


def test_workspace_sizes():
    assert wf.verify_workspace_bytes(0, V) == 0 and wf.verify_workspace_bytes(5, 0) == 0
    assert wf.route_workspace_bytes(0, 1024) == 0
    for rows in (1, 17, 544, 488, 4352, 4992):
        n = wf.verify_workspace_bytes(rows, V)
        assert n % 256 == 0 and n >= rows * 8
    assert wf.route_workspace_bytes(256, 1024) >= 256 * 1024 * 4


ALIGNED = 1 << 20   # a fake, suitably aligned device address: validation fails before it is used


def test_verify_chain_validation():
    f = wf.whiflash_verify_chain
    # (logits, dtype, B, K, V, stride, draft, al, bonus, rows, ws, ws_bytes, stream)
    assert f(None, 1, 1, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -1
    assert f(ALIGNED, 9, 1, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -3
    assert f(ALIGNED, 1, 1, -1, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -2
    assert f(ALIGNED, 1, 1, 1024, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -2
    assert f(ALIGNED, 1, 1, 16, V, V - 1, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -2
    assert f(ALIGNED, 1, 1, 16, 101, 101, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -4
    assert f(ALIGNED + 2, 1, 1, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -4
    assert f(ALIGNED, 1, 1, 16, V, V, None, ALIGNED, ALIGNED, None, ALIGNED, 1 << 20, None) == -1
    assert f(ALIGNED, 1, 1, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, None, 1 << 20, None) == -5
    assert f(ALIGNED, 1, 1, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 16, None) == -5
    assert f(ALIGNED, 1, 1, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED + 16, 1 << 20, None) == -5
    assert f(None, 1, 0, 16, V, V, None, None, None, None, None, 0, None) == 0   # B = 0: no-op


def test_verify_tree_validation():
    f = wf.whiflash_verify_tree
    args = [ALIGNED, 1, 8, 61, V, V, ALIGNED, ALIGNED, ALIGNED, 32000, ALIGNED, ALIGNED, None, None,
            ALIGNED, 1 << 20, None]
    bad = list(args); bad[3] = 0
    assert f(*bad) == -2
    bad = list(args); bad[3] = 1025
    assert f(*bad) == -2
    bad = list(args); bad[9] = 0
    assert f(*bad) == -2
    bad = list(args); bad[8] = None
    assert f(*bad) == -1
    bad = list(args); bad[15] = 100
    assert f(*bad) == -5


def test_verify_routed_validation():
    f = wf.whiflash_verify_routed
    args = [ALIGNED, 1, 128, V, V, ALIGNED, 4992, ALIGNED, 16, ALIGNED, 61, ALIGNED, ALIGNED,
            ALIGNED, 32000, ALIGNED, ALIGNED, None, None, ALIGNED, 1 << 20, None]
    bad = list(args); bad[5] = None
    assert f(*bad) == -1
    bad = list(args); bad[6] = -1
    assert f(*bad) == -2
    bad = list(args); bad[20] = 8
    assert f(*bad) == -5


def test_route_validation():
    f = wf.whiflash_route
    # (hidden, dtype, B, d, W1, b1, m, W2, b2, tau, dal, choice, ws, ws_bytes, stream)
    assert f(ALIGNED, 2, 4, 2560, ALIGNED, None, 1024, ALIGNED, None, 1.0, ALIGNED, ALIGNED, ALIGNED,
             1 << 24, None) == -3
    assert f(ALIGNED, 1, 4, 0, ALIGNED, None, 1024, ALIGNED, None, 1.0, ALIGNED, ALIGNED, ALIGNED,
             1 << 24, None) == -2
    assert f(None, 1, 4, 2560, ALIGNED, None, 1024, ALIGNED, None, 1.0, ALIGNED, ALIGNED, ALIGNED,
             1 << 24, None) == -1
    assert f(ALIGNED, 1, 4, 2560, ALIGNED, None, 1024, ALIGNED, None, 1.0, ALIGNED, ALIGNED, ALIGNED,
             64, None) == -5
    assert f(None, 1, 0, 2560, None, None, 1024, None, None, 1.0, None, None, None, 0, None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from drafter_routing_verification_amd import _binding
    monkeypatch.setattr(_binding, "_LIB", None)
    monkeypatch.setattr(_binding, "library_path", lambda: str(tmp_path / "libwhiflash.so"))
    with pytest.raises(_binding.WhiflashError):
        _binding.lib()


def test_entropy_validation():
    f = wf.whiflash_route_entropy
    # (logits, dtype, total_rows, V, stride, B, row0, rows_per_seq, pos, tau, H, choice, ws, ws_bytes, stream)
    ok = [ALIGNED, 1, 4992, V, V, 128, ALIGNED, 0, ALIGNED, 1.0, ALIGNED, ALIGNED, ALIGNED, 1 << 22, None]
    bad = list(ok); bad[8] = None
    assert f(*bad) == -1
    bad = list(ok); bad[6] = None; bad[7] = -1
    assert f(*bad) == -2
    bad = list(ok); bad[13] = 16
    assert f(*bad) == -5
    bad = list(ok); bad[1] = 3
    assert f(*bad) == -3
    bad = list(ok); bad[5] = 0
    assert f(*bad) == 0
    assert wf.entropy_workspace_bytes(128, V) >= 128 * 16 and wf.entropy_workspace_bytes(0, V) == 0


def test_catchup_validation():
    f = wf.whiflash_catchup_update
    assert f(4, None, ALIGNED, ALIGNED, ALIGNED, None, None, None) == -1
    assert f(-1, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, None, None) == -2
    assert f(0, None, None, None, None, None, None, None) == 0


def test_route_gather_validation():
    f = wf.whiflash_route_gather
    # (hidden_rows, dtype, total_rows, d, B, row0, rps, pos, W1, b1, m, W2, b2, tau, dal, ch, ws, ws_bytes, s)
    ok = [ALIGNED, 1, 4992, 2560, 128, ALIGNED, 0, ALIGNED, ALIGNED, None, 1024, ALIGNED, None, 1.0,
          ALIGNED, ALIGNED, ALIGNED, 1 << 26, None]
    bad = list(ok); bad[7] = None
    assert f(*bad) == -1
    bad = list(ok); bad[5] = None; bad[6] = -3
    assert f(*bad) == -2
    bad = list(ok); bad[17] = 64
    assert f(*bad) == -5


def test_verify_chain_early_exit_validation():
    f = wf.whiflash_verify_chain_early_exit
    ok = [ALIGNED, 1, 256, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 24, None]
    bad = list(ok); bad[6] = None
    assert f(*bad) == -1
    bad = list(ok); bad[3] = 1024
    assert f(*bad) == -2
    bad = list(ok); bad[5] = V - 8
    assert f(*bad) == -2
    bad = list(ok); bad[1] = 7
    assert f(*bad) == -3
    bad = list(ok); bad[0] = ALIGNED + 8
    assert f(*bad) == -4
    bad = list(ok); bad[11] = wf.early_exit_workspace_bytes(256, 16, V) - 1
    assert f(*bad) == -5
    bad = list(ok); bad[10] = ALIGNED + 64
    assert f(*bad) == -5
    bad = list(ok); bad[2] = 0
    assert f(*bad) == 0
    n = wf.early_exit_workspace_bytes(256, 16, V)
    assert n % 256 == 0 and n >= 256 * 4 + 256 * 17 * 8
    assert wf.early_exit_workspace_bytes(0, 16, V) == 0 and wf.early_exit_workspace_bytes(4, -1, V) == 0


def test_round_chain_validation():
    f = wf.whiflash_round_chain
    # (hidden, hdt, d, W1, b1, m, W2, b2, tau, dal, ch, logits, ldt, B, K, V, stride, draft,
    #  al, bonus, rows, ws, ws_bytes, stream)
    ok = [ALIGNED, 1, 2560, ALIGNED, None, 1024, ALIGNED, None, 1.0, ALIGNED, ALIGNED, ALIGNED, 1,
          256, 16, V, V, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, 1 << 30, None]
    bad = list(ok); bad[1] = 5
    assert f(*bad) == -3
    bad = list(ok); bad[14] = 1024
    assert f(*bad) == -2
    bad = list(ok); bad[17] = None
    assert f(*bad) == -1
    bad = list(ok); bad[0] = None
    assert f(*bad) == -1
    bad = list(ok); bad[22] = wf.round_chain_workspace_bytes(256, 1024, 16, V) - 1
    assert f(*bad) == -5
    bad = list(ok); bad[13] = 0
    assert f(*bad) == 0
    n = wf.round_chain_workspace_bytes(256, 1024, 16, V)
    assert n == wf.route_workspace_bytes(256, 1024) + wf.verify_workspace_bytes(256 * 17, V)


def test_argmax_sweep_plan_and_validation():
    # every chunk starts inside the row, chunks are 256-aligned, and they cover the row
    for rows, v in ((1, 7), (17, V), (4352, V), (4992, V), (3, 2049), (100000, 300)):
        chunks, elems = wf.argmax_sweep_plan(rows, v)
        assert chunks >= 1 and elems % 256 == 0
        assert (chunks - 1) * elems < v <= chunks * elems
        assert rows * chunks * 8 <= wf.verify_workspace_bytes(rows, v)
    with pytest.raises(wf.WhiflashError):
        wf.argmax_sweep_plan(0, V)
    f = wf.whiflash_argmax_sweep
    need = 4352 * wf.argmax_sweep_plan(4352, V)[0] * 8
    # (logits, dtype, rows, V, stride, partials, partials_bytes, stream)
    assert f(None, 1, 4352, V, V, ALIGNED, need, None) == -1
    assert f(ALIGNED, 7, 4352, V, V, ALIGNED, need, None) == -3
    assert f(ALIGNED, 1, -1, V, V, ALIGNED, need, None) == -2
    assert f(ALIGNED, 1, 4352, V, V - 8, ALIGNED, need, None) == -2
    assert f(ALIGNED + 8, 1, 4352, V, V, ALIGNED, need, None) == -4
    assert f(ALIGNED, 1, 4352, V, V, None, need, None) == -5
    assert f(ALIGNED, 1, 4352, V, V, ALIGNED, need - 8, None) == -5
    assert f(ALIGNED, 1, 4352, V, V, ALIGNED + 64, need, None) == -5
    assert f(None, 1, 0, V, V, None, 0, None) == 0   # rows = 0: no-op


def test_stream_read_validation():
    f = wf.whiflash_stream_read
    # (logits, dtype, rows, V, stride, sink, stream)
    assert f(None, 1, 0, V, V, None, None) == 0          # rows = 0: no-op
    assert f(None, 1, 4352, V, V, ALIGNED, None) == -1
    assert f(ALIGNED, 1, 4352, V, V, None, None) == -1
    assert f(ALIGNED, 5, 4352, V, V, ALIGNED, None) == -3
    assert f(ALIGNED, 1, 4352, V, V - 8, ALIGNED, None) == -2
    assert f(ALIGNED + 8, 1, 4352, V, V, ALIGNED, None) == -4


def test_workspace_queries_reject_row_counts_past_int32():
    # Sizes whose row count B*(K+1) or B*N exceeds INT32_MAX are rejected by the
    # calls, and their workspace queries answer 0 rather than overflow.
    big = 2**31 - 1
    assert wf.early_exit_workspace_bytes(2**21, 1023, V) == 0
    assert wf.early_exit_workspace_bytes(2, big, V) == 0
    assert wf.round_chain_workspace_bytes(2**21, 1024, 1023, V) == 0
    assert wf.round_chain_workspace_bytes(2, 1024, big, V) == 0
    assert wf.round_chain_early_exit_workspace_bytes(2**21, 1024, 1023, V) == 0
    assert wf.tree_early_exit_workspace_bytes(2**22, 1024, V) == 0
    assert wf.routed_early_exit_workspace_bytes(4, big, 16, 64, V) == 0
    assert wf.round_early_exit_workspace_bytes(4, 1024, big, 16, 64, V) == 0
    # Just inside the limit the queries still answer.
    assert wf.early_exit_workspace_bytes(2**21 - 1, 1023, V) > 0
    assert wf.tree_early_exit_workspace_bytes(2**21 - 1, 1024, V) > 0


def test_round_chain_noalloc_validation():
    """Argument checks of whiflash_round_chain_noalloc, all before any HIP call: those of
    whiflash_round_chain, then the fixed scratch's limit."""
    f = wf.whiflash_round_chain_noalloc
    A = ALIGNED
    # (hidden, hdt, d, W1, b1, m, W2, b2, tau, dal, choice, logits, ldt, B, K, V, stride, draft,
    #  al, bonus, rows, stream)
    ok = [A, 1, 2560, A, None, 1024, A, None, 1.0, A, A, A, 1, 256, 16, V, V, A, A, A, None, None]
    big = list(ok); big[13] = 1600                 # 1,600 chains need more than 8 MiB
    assert wf.round_chain_workspace_bytes(1600, 1024, 16, V) > (8 << 20)
    assert wf.round_chain_workspace_bytes(256, 1024, 16, V) <= (8 << 20)
    assert f(*big) == -7 and "scratch" in wf.status_string(-7)
    bad = list(big); bad[0] = None
    assert f(*bad) == -1                           # argument errors come first
    bad = list(ok); bad[12] = 5
    assert f(*bad) == -3
    bad = list(ok); bad[14] = 1024
    assert f(*bad) == -2
    bad = list(ok); bad[11] = A + 2
    assert f(*bad) == -4
    zero = list(ok); zero[13] = 0
    assert f(*zero) == 0                           # B = 0: no-op
