"""CPU oracle for the WhiFlash verify-and-route step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the method computes, used to check the HIP path.  Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may import
it; the product path never does and has no CPU fallback.  It shares no code
with the HIP library.

Every function is pinned by tests under ``tests/`` (brute force on tiny inputs,
closed forms, invariants, library special cases).  The pages print no worked
numerical example for any step, so no function is pinned to a printed value of
the pages; the router's shape is pinned to the parameter counts the paper's
router table prints.
"""

from .whiflash import (  # noqa: F401
    decode_logits,
    row_argmax,
    gelu,
    route,
    route_gather,
    entropy,
    route_entropy,
    verify_chain,
    verify_tree,
    tree_accepted,
    verify_routed,
    catchup_update,
    MALFORMED_AL,
    MALFORMED_BONUS,
)
