/*
 * whiflash.h -- C ABI of the MI355X (gfx950) verify-and-route library.
 *
 * One WhiFlash speculation round ends with three steps, all implemented here
 * as HIP kernels:
 *   route  : the neural router, a two-layer GELU MLP mapping the target's
 *            final hidden state to a predicted acceptance-length gain, and the
 *            hardware-aware threshold that turns it into a drafter choice;
 *   verify : greedy verification -- a full-vocabulary argmax of the target
 *            logits at every drafted position, then the accepted prefix of a
 *            DFlash block (chain) or the deepest accepted path of an EAGLE-3
 *            draft tree (after mapping draft-vocabulary ids to target ids);
 *   emit   : acceptance length (AL) and bonus token per sequence.
 * Sources: "WhiFlash: Accelerating Speculative Decoding with Token-Level
 * Cross-Paradigm Routing" (arXiv 2606.07710), sections 3.2 and 3.3 and
 * Appendix A; the "Qwen3-4B-EAGLE3" model card (fixed 32K draft vocabulary).
 *
 * Conventions shared by every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller.  The
 *     library keeps no pointer after the call returns and holds no state,
 *     apart from the fixed scratch of whiflash_round_chain_noalloc.
 *   - Calls are asynchronous on `stream` (0 = the default stream); none
 *     synchronises and none allocates.  Scratch memory comes from the
 *     caller's `workspace` (device memory of at least the size returned by
 *     the matching *_workspace_bytes function, 256-byte aligned).  Calls on
 *     different streams must use different workspaces.
 *   - Arrays are row-major.  Logits rows are `row_stride` elements apart;
 *     row_stride >= V, and the logits base address and row_stride * element
 *     size must both be multiples of 16 bytes.
 *   - Return value: WF_OK, or a negative wf_status for a problem the host
 *     can see (null pointer, bad size, dtype, alignment, workspace too
 *     small); nothing is launched then.  WF_ERR_LAUNCH reports a failed
 *     kernel launch.
 *   - Bad DATA never faults and has a defined result (identical in the CPU
 *     oracle): see each entry point.  Logits must not be NaN (the argmax of a
 *     row holding NaN is unspecified, but still an index in [0, V)).
 */
#ifndef WHIFLASH_H
#define WHIFLASH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of logits, hidden states and router weights. */
typedef enum { WF_F32 = 0, WF_BF16 = 1 } wf_dtype;

typedef enum {
  WF_OK = 0,
  WF_ERR_NULL = -1,      /* a required pointer is NULL                       */
  WF_ERR_SHAPE = -2,     /* a size is out of range                           */
  WF_ERR_DTYPE = -3,     /* dtype is not a wf_dtype value                    */
  WF_ERR_ALIGN = -4,     /* logits base or row stride not 16-byte aligned    */
  WF_ERR_WORKSPACE = -5, /* workspace NULL, misaligned or smaller than needed */
  WF_ERR_LAUNCH = -6,    /* the HIP runtime rejected a kernel launch         */
  WF_ERR_SCRATCH = -7,   /* the call needs more than the fixed scratch holds  */
  WF_ERR_RUNTIME = -8    /* a HIP runtime query (device, symbol) failed       */
} wf_status;

/* Largest K+1 (chain) or N (tree) rows per sequence the kernels accept. */
#define WHIFLASH_MAX_SEQ_ROWS 1024

/* Largest router hidden size d (and at most 65,535 sequences per router call). */
#define WHIFLASH_MAX_HIDDEN (1 << 24)

/* Human-readable name of a wf_status value (static string; host only). */
const char* whiflash_status_string(int32_t status);

/* Workspace bytes whiflash_route needs for batch B and router width m.
 * Returns 0 when B or m is not positive. Host only. */
size_t whiflash_route_workspace_bytes(int32_t B, int32_t m);

/* Workspace bytes the verify entry points need for `total_rows` logits rows
 * of V entries (chain: B*(K+1) rows, tree: B*N rows, routed: total_rows).
 * Returns 0 when total_rows or V is not positive. Host only. */
size_t whiflash_verify_workspace_bytes(int32_t total_rows, int32_t V);

/*
 * How the argmax sweep cuts `rows` rows of V entries: every row into *chunks
 * pieces, piece c covering entries [c * *chunk_elems, min(V, (c + 1) *
 * *chunk_elems)).  *chunk_elems is a multiple of 256.  Host only.  Returns
 * WF_ERR_SHAPE when rows < 1 or V < 1, WF_ERR_NULL when an output is NULL.
 */
int32_t whiflash_argmax_sweep_plan(int32_t rows, int32_t V, int32_t* chunks, int32_t* chunk_elems);

/*
 * The full-vocabulary argmax sweep alone: the first kernel of every verify
 * entry point (greedy verification takes the target's most likely token at
 * every drafted position; WhiFlash paper, section 3.2), launched by itself so
 * that its time can be measured without the acceptance kernel, or its
 * per-chunk results merged by the caller.
 *   logits [rows, V] with row_stride, as in the verify entry points.
 *   partials: device array of rows * chunks records {float max; int32 index},
 *     8 bytes each, record r * chunks + c for chunk c of row r (chunking from
 *     whiflash_argmax_sweep_plan): the chunk's largest value (bf16 widened
 *     exactly to float32) and the lowest row index holding it (an index into
 *     the row, in [0, V)).  partials_bytes >= rows * chunks * 8, base 256-byte
 *     aligned; whiflash_verify_workspace_bytes(rows, V) bytes always suffice.
 * rows == 0 is a no-op.  A chunk whose entries are all -inf reports -inf and
 * its first index.
 */
int32_t whiflash_argmax_sweep(const void* logits, int32_t dtype, int32_t rows, int32_t V,
                              int64_t row_stride, void* partials, size_t partials_bytes,
                              hipStream_t stream);

/*
 * A measurement aid, not a step of the method: the argmax sweep's reads
 * without its comparisons.  It reads the same whole 16-byte vectors of every
 * row as whiflash_argmax_sweep, cut into the same chunks and with the same
 * workgroups, launch order and load instructions, and folds them into an XOR.
 * The time it takes is a streaming-read ceiling for the sweep on the same
 * buffers.  Writes to *sink (device, one uint32) the XOR of the 32-bit words of
 * row 0's first chunk (entries [0, chunk_elems) of whiflash_argmax_sweep_plan,
 * whole vectors only).  rows == 0 is a no-op; otherwise logits and sink must
 * not be NULL.
 */
int32_t whiflash_stream_read(const void* logits, int32_t dtype, int32_t rows, int32_t V,
                             int64_t row_stride, uint32_t* sink, hipStream_t stream);

/*
 * Neural router + hardware-aware threshold (WhiFlash paper, section 3.3.2
 * "Neural Policy" and "Hardware-Aware Routing Decision"; Appendix A "Neural
 * Router Architecture"):
 *     z        = W1 h_b + b1                       (d -> m)
 *     g        = GELU(z) = z/2 * (1 + erf(z/sqrt 2)), dropout = identity
 *     dal[b]   = W2 . g + b2                       (m -> 1, predicted AL gain)
 *     choice[b]= 1 (EAGLE-3, autoregressive tree) if dal[b] > tau, else 0 (DFlash)
 *   hidden [B, d], W1 [m, d], W2 [m]: all of element type `dtype`.
 *   b1 [m] float32 or NULL (= 0); b2: pointer to one float32 or NULL (= 0).
 *   Accumulation, GELU and the second layer run in float32.
 *   delta_al [B] float32 and choice [B] int32 are written.
 * B == 0 is a no-op.  1 <= d <= WHIFLASH_MAX_HIDDEN, m >= 1, B <= 65535.  The
 * paper's router uses m = d/8; any m works.
 */
int32_t whiflash_route(const void* hidden, int32_t dtype, int32_t B, int32_t d,
                       const void* W1, const float* b1, int32_t m,
                       const void* W2, const float* b2, float tau,
                       float* delta_al, int32_t* choice,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same router fed from the hidden state at each sequence's final accepted
 * position (WhiFlash paper, section 3.3.2: the policy takes the final-layer
 * hidden state at the current decoding step; section 3.3.1: the final
 * accepted position).  hidden_rows [total_rows, d] holds the target's hidden
 * states for every verified row (the rows the verify calls read); sequence b
 * uses row row0[b] + pos[b], where row0 [B] is each sequence's first row (e.g.
 * the routed row_offsets) or NULL meaning b * rows_per_seq, and pos [B] is the
 * accepted position within the sequence (best_node from the verify calls, or
 * accept_len - 1 for a chain).  A negative pos or a row outside
 * [0, total_rows) gives delta_al = NaN and choice 0.  Other arguments, the
 * workspace (whiflash_route_workspace_bytes(B, m)) and the arithmetic are
 * those of whiflash_route.
 */
int32_t whiflash_route_gather(const void* hidden_rows, int32_t dtype, int32_t total_rows,
                              int32_t d, int32_t B, const int32_t* row0, int32_t rows_per_seq,
                              const int32_t* pos, const void* W1, const float* b1, int32_t m,
                              const void* W2, const float* b2, float tau, float* delta_al,
                              int32_t* choice, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Greedy verification of DFlash blocks (WhiFlash paper, section 3.2: the
 * drafted block is verified in parallel and decoding continues from the last
 * accepted token; section 4 "Metrics": AL counts tokens per round).
 *   logits: B*(K+1) rows; row b*(K+1)+i is the target's prediction after the
 *           first i draft tokens of sequence b (row K follows a full match).
 *   draft [B, K] int32 target ids.
 *   t[r] = lowest index holding the maximum of row r.
 *   n = first i < K with draft[b,i] != t[b*(K+1)+i], else K;
 *   accept_len[b] = n + 1 (in [1, K+1]); bonus[b] = t[b*(K+1)+n].
 *   row_argmax [B*(K+1)] (t) is written when not NULL.
 * A draft id outside [0, V) never matches.  B == 0 is a no-op; K >= 0;
 * K + 1 <= WHIFLASH_MAX_SEQ_ROWS.
 */
int32_t whiflash_verify_chain(const void* logits, int32_t dtype, int32_t B, int32_t K, int32_t V,
                              int64_t row_stride, const int32_t* draft,
                              int32_t* accept_len, int32_t* bonus, int32_t* row_argmax,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes whiflash_verify_chain_early_exit needs (host-only; 0 when
 * B <= 0, K < 0, V <= 0 or B * (K + 1) exceeds INT32_MAX). */
size_t whiflash_early_exit_workspace_bytes(int32_t B, int32_t K, int32_t V);

/*
 * DFlash chain verification that reads only the rows it needs (WhiFlash
 * paper, section 3.2: decoding continues from the last accepted token, so the
 * rows after the first rejected draft affect neither AL nor the bonus token).
 * Arguments, layouts, data rules and errors are those of whiflash_verify_chain,
 * and accept_len and bonus are identical to its results.  row_argmax (when not
 * NULL) holds t for rows 0..n of each sequence and -1 for the rows after n.
 * Rows of a sequence after its first mismatch may be skipped in whole or in
 * part, so the logits bytes read depend on the data (at least rows 0..n).
 * Workspace: whiflash_early_exit_workspace_bytes(B, K, V) bytes, 256-byte
 * aligned; it holds per-sequence flags that the call clears itself, so two
 * calls that share a workspace must not overlap in time.
 */
int32_t whiflash_verify_chain_early_exit(const void* logits, int32_t dtype, int32_t B, int32_t K,
                                         int32_t V, int64_t row_stride, const int32_t* draft,
                                         int32_t* accept_len, int32_t* bonus, int32_t* row_argmax,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * Greedy verification of EAGLE-3 draft trees with the draft-to-target map
 * (WhiFlash paper, section 3.2: a tree of candidate tokens is verified;
 * "Qwen3-4B-EAGLE3" card: draft ids come from a fixed 32K vocabulary).
 *   logits: B*N rows; row b*N+u is the target's prediction after node u of
 *           tree b.  Node 0 is the root (the last verified token).
 *   parent [B, N] int32: parent[b,0] is ignored; node u >= 1 hangs under
 *           parent[b,u], which must lie in [0, u) (else u is unreachable).
 *   draft_ids [B, N] int32 draft-vocabulary ids (entry 0 ignored).
 *   d2t [Vd] int32 absolute target id of each draft id.
 *   Node u >= 1 is accepted iff its parent p is accepted and
 *   d2t[draft_ids[b,u]] == t[b*N+p]; ids outside [0, Vd) and table entries
 *   outside [0, V) never match.  best = deepest accepted node (lowest index
 *   among equally deep ones); accept_len[b] = depth(best) + 1,
 *   bonus[b] = t[b*N+best], best_node[b] = best (when not NULL).
 *   row_argmax [B*N] is written when not NULL.
 * B == 0 is a no-op; 1 <= N <= WHIFLASH_MAX_SEQ_ROWS; Vd >= 1.
 */
int32_t whiflash_verify_tree(const void* logits, int32_t dtype, int32_t B, int32_t N, int32_t V,
                             int64_t row_stride, const int32_t* parent, const int32_t* draft_ids,
                             const int32_t* d2t, int32_t Vd,
                             int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                             int32_t* row_argmax,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Routed mixed batch: each sequence is verified by the drafter its router
 * choice selected (WhiFlash paper, section 3.3: one routing decision per
 * sequence and speculation round).
 *   logits: total_rows packed rows; sequence b owns rows
 *           [row_offsets[b], row_offsets[b+1]).
 *   row_offsets [B+1] int32 (device); total_rows is the host's copy of the
 *           number of packed rows (the sweep covers rows [0, total_rows)).
 *   choice [B] int32 (e.g. the output of whiflash_route): 0 = DFlash chain
 *           needing K+1 rows, verified with chain_draft[b, 0..K-1];
 *           1 = EAGLE-3 tree needing N rows, verified with parent[b,:],
 *           draft_ids[b,:] and d2t as in whiflash_verify_tree.
 *   chain_draft [B, K], parent [B, N], draft_ids [B, N]: rows belonging to
 *           sequences of the other kind are not read.
 *   A sequence whose offsets are decreasing or outside [0, total_rows],
 *   whose row count does not match its choice, or whose choice is neither 0
 *   nor 1 gets accept_len 0, bonus -1, best_node -1 (AL 0 cannot occur
 *   otherwise).  For chain sequences best_node = accept_len - 1.
 *   row_argmax [total_rows] is written when not NULL, for every row covered
 *   by some sequence's offsets range.
 * B == 0 is a no-op; total_rows >= 0; K >= 0; K+1 and N <= WHIFLASH_MAX_SEQ_ROWS.
 */
int32_t whiflash_verify_routed(const void* logits, int32_t dtype, int32_t B, int32_t V,
                               int64_t row_stride, const int32_t* row_offsets, int32_t total_rows,
                               const int32_t* choice,
                               int32_t K, const int32_t* chain_draft,
                               int32_t N, const int32_t* parent, const int32_t* draft_ids,
                               const int32_t* d2t, int32_t Vd,
                               int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                               int32_t* row_argmax,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes whiflash_round_routed needs (router and sweep regions).
 * Returns 0 when B, m or V is not positive. Host only. */
size_t whiflash_round_workspace_bytes(int32_t B, int32_t m, int32_t total_rows, int32_t V);

/*
 * One routed speculation round: whiflash_route (hidden, W1, b1, W2, b2, tau ->
 * delta_al, choice) followed by whiflash_verify_routed with that choice, with
 * the same arguments, results and error codes as the two calls (hidden_dtype
 * is the router's element type, logits_dtype the logits').  It runs in three
 * launches instead of four: router stage 1, the argmax sweep, then one kernel
 * per sequence that finishes the router and verifies the sequence.  Router
 * stage 1 and the sweep share one launch (two in all) when the hidden states
 * and W1 are 16-byte aligned with d a multiple of 16 bytes of elements and
 * either there are at most 8 sequences (the router's GEMV path) or the bf16
 * router is small (at most 2,048 64-column chunk loads of its MFMA tiles, e.g.
 * up to 64 sequences at 2560 -> 1024).  Callers that cannot fuse the two steps
 * (e.g. a different stream for each) use the separate entry points.
 */
int32_t whiflash_round_routed(const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, const float* b2,
                              float tau, float* delta_al, int32_t* choice, const void* logits,
                              int32_t logits_dtype, int32_t B, int32_t V, int64_t row_stride,
                              const int32_t* row_offsets, int32_t total_rows, int32_t K,
                              const int32_t* chain_draft, int32_t N, const int32_t* parent,
                              const int32_t* draft_ids, const int32_t* d2t, int32_t Vd,
                              int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                              int32_t* row_argmax, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Lazy catch-up bookkeeping (WhiFlash paper, section 3.4 "Lazy Catch-up": the
 * inactive drafter defers its KV-cache updates; the tokens accepted while it
 * is inactive are its backlog, prefilled in one batch when a switch to it is
 * committed).  Per sequence b, after a round verified with drafter
 * cur_choice[b] (0 DFlash, 1 EAGLE-3) that accepted accept_len[b] tokens, and
 * with next_choice[b] chosen for the next round:
 *     backlog[b][1 - cur] += accept_len[b]           (if accept_len[b] > 0)
 *     if next != cur: catchup_len[b] = backlog[b][next]; backlog[b][next] = 0;
 *                     switch_flag[b] = 1
 *     else:           catchup_len[b] = 0; switch_flag[b] = 0
 * backlog [B, 2] int32 is updated in place (start from zeros).  A choice
 * outside {0, 1} leaves the sequence unchanged with no switch.
 * switch_flag [B] and catchup_len [B] may be NULL.  No workspace.
 */
int32_t whiflash_catchup_update(int32_t B, const int32_t* cur_choice, const int32_t* accept_len,
                                const int32_t* next_choice, int32_t* backlog, int32_t* switch_flag,
                                int32_t* catchup_len, hipStream_t stream);

/* Workspace bytes whiflash_route_entropy needs for B sequences and rows of V
 * entries.  Returns 0 when B or V is not positive. Host only. */
size_t whiflash_entropy_workspace_bytes(int32_t B, int32_t V);

/*
 * WhiFlash-Entropy policy (WhiFlash paper, section 3.3.1 "Runtime-Informed
 * Policy"): for each sequence b, the entropy in nats of the softmax of the
 * logits row at its final accepted position,
 *     H[b] = -sum_x p(x) log p(x),  p = softmax(row),
 * and the decision choice[b] = 1 (EAGLE-3) if H[b] > tau, else 0 (DFlash).
 *   logits: total_rows packed rows of V entries, row_stride apart (the rows the
 *           verify entry points read).
 *   The selected row of sequence b is row0[b] + pos[b], where row0 is a [B]
 *   device array of each sequence's first row (e.g. the routed row_offsets),
 *   or NULL meaning row0[b] = b * rows_per_seq; pos [B] is the position within
 *   the sequence (the best_node output of the verify calls, or accept_len - 1
 *   for a chain).  A negative pos or a row outside [0, total_rows) gives
 *   H = NaN and choice 0.
 *   entropy [B] float32 and choice [B] int32 are written.  The reduction runs
 *   in float32 with a fixed merge order (bitwise reproducible).
 * Precondition: the selected rows hold finite values.  B == 0 is a no-op.
 */
int32_t whiflash_route_entropy(const void* logits, int32_t dtype, int32_t total_rows, int32_t V,
                               int64_t row_stride, int32_t B, const int32_t* row0,
                               int32_t rows_per_seq, const int32_t* pos, float tau,
                               float* entropy, int32_t* choice,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of whiflash_verify_tree_early_exit (host-only; 0 on bad sizes). */
size_t whiflash_tree_early_exit_workspace_bytes(int32_t B, int32_t N, int32_t V);

/*
 * EAGLE-3 tree verification that reads only the rows it needs (WhiFlash
 * paper, section 3.2: a tree of candidate tokens is verified and decoding
 * continues from the deepest accepted node, so only the rows of accepted
 * nodes decide the acceptance length, the best node and the bonus token).
 * Arguments, layouts, data rules and errors are those of whiflash_verify_tree,
 * and accept_len, bonus and best_node are identical to its results.
 * row_argmax (when not NULL) holds t for the rows of accepted nodes and -1
 * for every other row.  Rows of nodes that are not accepted may be skipped in
 * whole or in part.  Workspace: whiflash_tree_early_exit_workspace_bytes(B, N,
 * V) bytes, 256-byte aligned, contents ignored on entry; two calls that share
 * a workspace must not overlap in time.
 */
int32_t whiflash_verify_tree_early_exit(const void* logits, int32_t dtype, int32_t B, int32_t N,
                                        int32_t V, int64_t row_stride, const int32_t* parent,
                                        const int32_t* draft_ids, const int32_t* d2t, int32_t Vd,
                                        int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                                        int32_t* row_argmax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of whiflash_verify_routed_early_exit (host-only; 0 on bad sizes). */
size_t whiflash_routed_early_exit_workspace_bytes(int32_t B, int32_t K, int32_t N,
                                                  int32_t total_rows, int32_t V);

/*
 * Routed verification that reads only the rows it needs: each DFlash chain up
 * to its first mismatch, each EAGLE-3 tree along its accepted nodes (same
 * passages as whiflash_verify_chain_early_exit and
 * whiflash_verify_tree_early_exit).  Arguments, layouts, data rules and errors
 * are those of whiflash_verify_routed; accept_len, bonus and best_node are
 * identical to its results (malformed sequences: AL 0, bonus -1, best -1, and
 * none of their rows are read).  row_argmax (when not NULL) holds t for the
 * rows of accepted nodes and -1 for the other rows of in-range sequences;
 * where the row ranges of two sequences overlap, a shared row's entry is
 * unspecified.  Workspace: whiflash_routed_early_exit_workspace_bytes(B, K, N,
 * total_rows, V) bytes, 256-byte aligned, contents ignored on entry; calls
 * sharing a workspace must not overlap in time.
 */
int32_t whiflash_verify_routed_early_exit(const void* logits, int32_t dtype, int32_t B, int32_t V,
                                          int64_t row_stride, const int32_t* row_offsets,
                                          int32_t total_rows, const int32_t* choice, int32_t K,
                                          const int32_t* chain_draft, int32_t N,
                                          const int32_t* parent, const int32_t* draft_ids,
                                          const int32_t* d2t, int32_t Vd, int32_t* accept_len,
                                          int32_t* bonus, int32_t* best_node, int32_t* row_argmax,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* Workspace bytes of whiflash_round_routed_early_exit (host-only; 0 on bad sizes). */
size_t whiflash_round_early_exit_workspace_bytes(int32_t B, int32_t m, int32_t K, int32_t N,
                                                 int32_t total_rows, int32_t V);

/*
 * One routed round with the early-exit verification: whiflash_route followed
 * by whiflash_verify_routed_early_exit with the router's choice, in four
 * launches (router stage 1; router finish + per-sequence preparation; the
 * node-major sweep; the acceptance).  Arguments and errors are those of
 * whiflash_round_routed; delta_al, choice, accept_len, bonus and best_node are
 * those of the two calls made in turn; row_argmax as in
 * whiflash_verify_routed_early_exit.  Workspace:
 * whiflash_round_early_exit_workspace_bytes(B, m, K, N, total_rows, V) bytes.
 */
int32_t whiflash_round_routed_early_exit(
    const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1, const float* b1, int32_t m,
    const void* W2, const float* b2, float tau, float* delta_al, int32_t* choice,
    const void* logits, int32_t logits_dtype, int32_t B, int32_t V, int64_t row_stride,
    const int32_t* row_offsets, int32_t total_rows, int32_t K, const int32_t* chain_draft,
    int32_t N, const int32_t* parent, const int32_t* draft_ids, const int32_t* d2t, int32_t Vd,
    int32_t* accept_len, int32_t* bonus, int32_t* best_node, int32_t* row_argmax, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of whiflash_verify_routed_entropy (host-only; 0 on bad sizes). */
size_t whiflash_verify_routed_entropy_workspace_bytes(int32_t B, int32_t total_rows, int32_t V);

/*
 * One round of the WhiFlash-Entropy policy (WhiFlash paper, section 3.3.1:
 * the entropy of the target's next-token distribution at the final accepted
 * position decides the next drafter): whiflash_verify_routed, then the entropy
 * of the softmax of each sequence's accepted row (its first row + best node)
 * and its threshold, as whiflash_route_entropy computes them.  Arguments,
 * layouts and errors are those of whiflash_verify_routed plus:
 *   tau_entropy  threshold on H (nats);
 *   entropy [B] float32  H of the accepted row (NaN for malformed sequences);
 *   next_choice [B] int32  1 (EAGLE-3) iff H > tau_entropy, else 0.
 * best_node may be NULL (the workspace then holds it).  Results equal those
 * of whiflash_verify_routed followed by whiflash_route_entropy(row0 =
 * row_offsets, pos = best_node).  Finite logits are required for H.
 * Workspace: whiflash_verify_routed_entropy_workspace_bytes(B, total_rows, V)
 * bytes, 256-byte aligned.
 */
int32_t whiflash_verify_routed_entropy(const void* logits, int32_t dtype, int32_t B, int32_t V,
                                       int64_t row_stride, const int32_t* row_offsets,
                                       int32_t total_rows, const int32_t* choice, int32_t K,
                                       const int32_t* chain_draft, int32_t N,
                                       const int32_t* parent, const int32_t* draft_ids,
                                       const int32_t* d2t, int32_t Vd, float tau_entropy,
                                       int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                                       int32_t* row_argmax, float* entropy, int32_t* next_choice,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Workspace bytes of whiflash_round_chain (host-only; 0 on bad sizes). */
size_t whiflash_round_chain_workspace_bytes(int32_t B, int32_t m, int32_t K, int32_t V);

/*
 * One DFlash round over a chain-only batch (WhiFlash paper, sections 3.2 and
 * 3.3): whiflash_route on hidden [B, d] (its choice is the drafter for the
 * next round) and whiflash_verify_chain on this round's logits and drafts, in
 * three launches instead of four (router stage 1; the argmax sweep; one
 * kernel per sequence that finishes the router and scans the chain), or two
 * when router stage 1 and the sweep share a launch (under the same conditions
 * as in whiflash_round_routed).
 * Arguments, layouts and errors are those of the two calls; delta_al, choice,
 * accept_len, bonus and row_argmax equal theirs.  Workspace:
 * whiflash_round_chain_workspace_bytes(B, m, K, V) bytes, 256-byte aligned.
 */
int32_t whiflash_round_chain(const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1,
                             const float* b1, int32_t m, const void* W2, const float* b2,
                             float tau, float* delta_al, int32_t* choice, const void* logits,
                             int32_t logits_dtype, int32_t B, int32_t K, int32_t V,
                             int64_t row_stride, const int32_t* draft, int32_t* accept_len,
                             int32_t* bonus, int32_t* row_argmax, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of whiflash_round_chain_early_exit (host-only; 0 on bad sizes). */
size_t whiflash_round_chain_early_exit_workspace_bytes(int32_t B, int32_t m, int32_t K, int32_t V);

/*
 * whiflash_round_chain with the early-exit verification: whiflash_route and
 * whiflash_verify_chain_early_exit in three launches (router stage 1, which
 * also clears the mismatch flags; the early-exit sweep; acceptance + router
 * finish).  Arguments and errors are those of whiflash_round_chain;
 * delta_al, choice, accept_len, bonus and row_argmax equal those of the two
 * calls made in turn.  Workspace:
 * whiflash_round_chain_early_exit_workspace_bytes(B, m, K, V) bytes, 256-byte
 * aligned; calls sharing a workspace must not overlap in time.
 */
int32_t whiflash_round_chain_early_exit(const void* hidden, int32_t hidden_dtype, int32_t d,
                                        const void* W1, const float* b1, int32_t m, const void* W2,
                                        const float* b2, float tau, float* delta_al,
                                        int32_t* choice, const void* logits, int32_t logits_dtype,
                                        int32_t B, int32_t K, int32_t V, int64_t row_stride,
                                        const int32_t* draft, int32_t* accept_len, int32_t* bonus,
                                        int32_t* row_argmax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* Bytes of the fixed device scratch of whiflash_round_chain_noalloc (per GPU). */
#define WHIFLASH_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * whiflash_round_chain for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, layouts, results and error codes are those of whiflash_round_chain,
 * without the workspace: the round's scratch is a fixed array of
 * WHIFLASH_NOALLOC_SCRATCH_BYTES bytes of device memory inside the library, one
 * copy per GPU, held until the process ends.  The call allocates nothing.
 *   - A round whose whiflash_round_chain_workspace_bytes(B, m, K, V) exceeds
 *     WHIFLASH_NOALLOC_SCRATCH_BYTES returns WF_ERR_SCRATCH and launches
 *     nothing (past 1,367 sequences at K = 16, V = 151,936, m = 1024; 256
 *     sequences need 2.6 MB).
 *   - The GPU is the stream's device (the current device for stream 0).  The
 *     first call on each GPU looks up that GPU's address of the array
 *     (WF_ERR_RUNTIME if the runtime cannot give it); later calls reuse it.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents.  Calls that overlap in time on one GPU (different
 *     streams, or host threads) race on it and must be serialised by the
 *     caller.  Nothing in it needs clearing: each call writes every byte it
 *     reads before reading it.
 */
int32_t whiflash_round_chain_noalloc(const void* hidden, int32_t hidden_dtype, int32_t d,
                                     const void* W1, const float* b1, int32_t m, const void* W2,
                                     const float* b2, float tau, float* delta_al, int32_t* choice,
                                     const void* logits, int32_t logits_dtype, int32_t B,
                                     int32_t K, int32_t V, int64_t row_stride,
                                     const int32_t* draft, int32_t* accept_len, int32_t* bonus,
                                     int32_t* row_argmax, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WHIFLASH_H */
