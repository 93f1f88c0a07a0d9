"""Python binding of libwhiflash, the MI355X verify-and-route library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/whiflash.h``.  Tensors must be torch device tensors on a
ROCm GPU; outputs are allocated here when not supplied.  There is no CPU
fallback: if the shared library is missing the import of the binding fails.

Entry points (same names as the C ABI):
    route(hidden, W1, b1, W2, b2, tau)                    -> (delta_al, choice)
    route_gather(hidden_rows, pos, W1, b1, W2, b2, tau, row0=None, rows_per_seq=0)
                                                          -> (delta_al, choice)
    argmax_sweep(logits)          the argmax sweep kernel alone -> (chunk max, chunk index)
    stream_read(logits)           measurement aid: the sweep's reads alone -> sink word
    verify_chain(logits, draft)                           -> (accept_len, bonus, row_argmax)
    verify_chain_early_exit(logits, draft)                -> (accept_len, bonus, row_argmax)
    verify_tree_early_exit, verify_routed_early_exit, round_routed_early_exit: same arguments
        and results as verify_tree, verify_routed, round_routed; only the rows of accepted
        nodes are read, and row_argmax is -1 for the others
    verify_tree(logits, parent, draft_ids, d2t)           -> (accept_len, bonus, best_node, row_argmax)
    verify_routed(logits, row_offsets, total_rows, choice, chain_draft, parent, draft_ids, d2t)
                                                          -> (accept_len, bonus, best_node, row_argmax)
    route_entropy(logits, pos, tau, row0=None, rows_per_seq=0)  -> (entropy, choice)
    verify_routed_entropy(logits, row_offsets, total_rows, choice, chain_draft, parent, draft_ids,
                          d2t, tau)   verify_routed + the entropy policy at the accepted rows
                          -> (accept_len, bonus, best_node, row_argmax, entropy, next_choice)
    catchup_update(cur_choice, accept_len, next_choice, backlog)  -> (switch_flag, catchup_len)
    round_chain(hidden, W1, b1, W2, b2, tau, logits, draft)   route + verify_chain fused
                 -> (delta_al, choice, accept_len, bonus, row_argmax)
    round_chain_noalloc(hidden, W1, b1, W2, b2, tau, logits, draft)   the same, with the
                 library's fixed device scratch in place of a workspace
    round_routed(hidden, W1, b1, W2, b2, tau, logits, row_offsets, total_rows, chain_draft,
                 parent, draft_ids, d2t)   route + verify_routed fused
                 -> (delta_al, choice, accept_len, bonus, best_node, row_argmax)
"""

from ._binding import (  # noqa: F401
    WF_F32,
    WF_BF16,
    WF_OK,
    WhiflashError,
    lib,
    library_path,
    status_string,
    route_workspace_bytes,
    verify_workspace_bytes,
    argmax_sweep,
    argmax_sweep_plan,
    whiflash_argmax_sweep,
    stream_read,
    whiflash_stream_read,
    route,
    route_gather,
    whiflash_route_gather,
    verify_chain,
    verify_tree,
    verify_chain_early_exit,
    verify_tree_early_exit,
    verify_routed_early_exit,
    round_routed_early_exit,
    tree_early_exit_workspace_bytes,
    routed_early_exit_workspace_bytes,
    round_early_exit_workspace_bytes,
    whiflash_verify_tree_early_exit,
    whiflash_verify_routed_early_exit,
    whiflash_round_routed_early_exit,
    early_exit_workspace_bytes,
    whiflash_verify_chain_early_exit,
    verify_routed,
    route_entropy,
    verify_routed_entropy,
    verify_routed_entropy_workspace_bytes,
    whiflash_verify_routed_entropy,
    entropy_workspace_bytes,
    catchup_update,
    whiflash_catchup_update,
    round_routed,
    round_chain,
    round_chain_noalloc,
    whiflash_round_chain_noalloc,
    round_chain_workspace_bytes,
    round_chain_early_exit,
    round_chain_early_exit_workspace_bytes,
    whiflash_round_chain_early_exit,
    whiflash_round_chain,
    round_workspace_bytes,
    whiflash_round_routed,
    whiflash_route_entropy,
    whiflash_route,
    whiflash_verify_chain,
    whiflash_verify_tree,
    whiflash_verify_routed,
)
