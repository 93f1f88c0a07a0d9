// Internal declarations shared by the HIP translation units of libwhiflash.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "whiflash.h"

namespace wf {

constexpr int kThreads = 256;          // every kernel runs 256-thread workgroups (4 wave64s)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxSeqRows = WHIFLASH_MAX_SEQ_ROWS;
constexpr int kRowsPerThread = kMaxSeqRows / kThreads;
// Largest router hidden size (keeps every column index of a hidden row far inside int).
constexpr int32_t kMaxHidden = WHIFLASH_MAX_HIDDEN;

// Partial result of the argmax sweep over one chunk of one row: the chunk's
// maximum and the lowest index holding it.
struct Partial {
  float val;
  int32_t idx;
};

// How the sweep cuts rows into chunks.  `chunk` is a multiple of 256 elements,
// so every chunk starts on a 16-byte vector boundary for both element types.
struct SweepPlan {
  int32_t splits;  // chunks per row
  int32_t chunk;   // elements per chunk (last chunk of a row may be shorter)
};

SweepPlan sweep_plan(int32_t rows, int32_t V);
// Whether a sweep launch of `blocks` workgroups issues each thread's whole batch of
// loads at once (small launches) or one load at a time.
bool sweep_batched(int64_t blocks);

// Row of sequence b selected as row0[b] + pos[b] (row0 NULL: b * rows_per_seq),
// or -1 when pos[b] < 0 or the row falls outside [0, total_rows).
__device__ inline int64_t select_row(const int32_t* row0, int32_t rows_per_seq, const int32_t* pos,
                                     int32_t total_rows, int b) {
  const int p = pos[b];
  const int64_t r =
      (row0 ? static_cast<int64_t>(row0[b]) : static_cast<int64_t>(b) * rows_per_seq) + p;
  return (p >= 0 && r >= 0 && r < total_rows) ? r : -1;
}

// An int32 array a launch zeroes on the side (its first workgroup), so a later
// launch on the same stream finds it cleared without a launch of its own.
struct ZeroFill {
  int32_t* p;
  int32_t n;
};

__device__ inline void zero_fill_first_block(const ZeroFill& z) {
  if (z.p && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < z.n; i += blockDim.x) z.p[i] = 0;
}

// Which hidden row feeds sequence b of the router: b itself (pos == NULL), or
// the row selected by (row0, rows_per_seq, pos) among total_rows rows.
struct HiddenSel {
  const int32_t* row0;
  const int32_t* pos;
  int32_t rows_per_seq;
  int32_t total_rows;
};

__device__ inline int64_t hidden_row(const HiddenSel& s, int b) {
  return s.pos ? select_row(s.row0, s.rows_per_seq, s.pos, s.total_rows, b) : b;
}

hipError_t launch_sweep(const void* logits, int dtype, int64_t row_stride, int32_t rows, int32_t V,
                        SweepPlan plan, Partial* part, hipStream_t stream);
// The sweep's reads alone (same chunks, workgroups and loads, no comparisons);
// writes one word derived from chunk 0 of row 0 to *sink.
hipError_t launch_stream_read(const void* logits, int dtype, int64_t row_stride, int32_t rows,
                              int32_t V, SweepPlan plan, unsigned* sink, hipStream_t stream);


// Early-exit verification of trees and routed batches (see early_exit.hip).
constexpr int kMaxMaskWords = (kMaxSeqRows + 63) / 64;

struct EeTreeArgs {
  int B, Rmax, W;              // sequences, rows of the longest sequence, 64-bit mask words
  const int32_t* row_offsets;  // [B+1] device, or NULL: sequence b at rows [b*N, b*N+N)
  const int32_t* choice;       // [B] device, or NULL: every sequence is a tree
  int total_rows, K, N, V, Vd;
  const int32_t* chain_draft;  // [B, K]
  const int32_t* parent;       // [B, N]
  const int32_t* draft_ids;    // [B, N]
  const int32_t* d2t;          // [Vd]
  const unsigned char* logits;
  int64_t row_bytes;
  int dtype;
  unsigned long long* mask;    // [B][W] rejected nodes
  unsigned long long* anc;     // [B][Rmax][W] ancestor-or-self masks
  int32_t* rowmap;             // [Rmax][B] global row of node u of sequence b, or -1
  int4* edge;                  // [B][Rmax] (parent, target token, parent-row logit bits, valid)
  int32_t* seq_off;            // [B+1] written for tree-only batches
  int32_t* seq_choice;         // [B] written for tree-only batches
};

// Byte offsets of the regions of an early-exit tree / routed workspace.
struct EeTreeWs {
  size_t mask, anc, rowmap, edge, seq_off, seq_choice, part, total;
};

EeTreeWs ee_tree_workspace(int32_t B, int32_t Rmax, int32_t total_rows, int32_t V, size_t align);
EeTreeArgs ee_tree_args(char* ws, const EeTreeWs& off, int32_t B, int32_t Rmax, const void* logits,
                        int dtype, int64_t row_stride, int32_t V, const int32_t* row_offsets,
                        const int32_t* choice, int32_t total_rows, int32_t K,
                        const int32_t* chain_draft, int32_t N, const int32_t* parent,
                        const int32_t* draft_ids, const int32_t* d2t, int32_t Vd);
hipError_t launch_ee_tree_prep(const EeTreeArgs& a, hipStream_t stream);
struct RouterPlan;
hipError_t launch_ee_round_prep(const EeTreeArgs& a, int hidden_dtype, const RouterPlan& plan,
                                const float* zp, int32_t m, const float* b1, const void* W2,
                                const float* b2, float tau, float* delta_al, int32_t* choice,
                                hipStream_t stream);
hipError_t launch_ee_tree_sweep(const EeTreeArgs& a, SweepPlan plan, Partial* part,
                                hipStream_t stream);

// Early-exit chain verification: chunk plan, and clear + sweep + accept launches.
// flags holds B int32 (cleared by the call), part B * (K + 1) * plan.splits partials.
SweepPlan early_exit_plan(int32_t B, int32_t V);
hipError_t launch_early_exit_chain(const void* logits, int dtype, int64_t row_stride, int32_t B,
                                   int32_t K, int32_t V, SweepPlan plan, const int32_t* draft,
                                   int* flags, Partial* part, int32_t* accept_len, int32_t* bonus,
                                   int32_t* row_argmax, hipStream_t stream);
// The early-exit chain round: sweep, then acceptance + router finish.  The
// flags must already be zero (router stage 1 clears them on the side).
struct RouterPlan;
hipError_t launch_early_exit_round(const void* logits, int dtype, int64_t row_stride, int32_t B,
                                   int32_t K, int32_t V, SweepPlan plan, const int32_t* draft,
                                   int* flags, Partial* part, int hidden_dtype,
                                   const RouterPlan& rplan, const float* zp, int32_t m,
                                   const float* b1, const void* W2, const float* b2, float tau,
                                   float* delta_al, int32_t* choice, int32_t* accept_len,
                                   int32_t* bonus, int32_t* row_argmax, hipStream_t stream);

// Every check of whiflash_round_chain's arguments except the workspace's (WF_OK or a
// negative status; runs no HIP call).
int32_t round_chain_check(const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1,
                          int32_t m, const void* W2, const float* delta_al, const int32_t* choice,
                          const void* logits, int32_t logits_dtype, int32_t B, int32_t K, int32_t V,
                          int64_t row_stride, const int32_t* draft, const int32_t* accept_len,
                          const int32_t* bonus);

hipError_t launch_finalize_chain(const Partial* part, int32_t splits, int32_t B, int32_t K,
                                 const int32_t* draft, int32_t* accept_len, int32_t* bonus,
                                 int32_t* row_argmax, hipStream_t stream);

hipError_t launch_finalize_tree(const Partial* part, int32_t splits, int32_t B, int32_t N, int32_t V,
                                const int32_t* parent, const int32_t* draft_ids, const int32_t* d2t,
                                int32_t Vd, int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                                int32_t* row_argmax, hipStream_t stream);

hipError_t launch_finalize_routed(bool early, const Partial* part, int32_t splits, int32_t B, int32_t V,
                                  const int32_t* row_offsets, int32_t total_rows,
                                  const int32_t* choice, int32_t K, const int32_t* chain_draft,
                                  int32_t N, const int32_t* parent, const int32_t* draft_ids,
                                  const int32_t* d2t, int32_t Vd, int32_t* accept_len,
                                  int32_t* bonus, int32_t* best_node, int32_t* row_argmax,
                                  hipStream_t stream);

// Router: stage 1 writes pre-activation partial sums zp[s][b][j] over `slices`
// slices of the hidden size; stage 2 finishes each sequence.
constexpr int32_t kMaxRouterSlices = 8;

struct RouterPlan {
  bool mfma;       // bf16 MFMA tiles (else the wave-per-unit GEMV, one slice)
  int32_t slices;  // slices of the hidden size (workgroups along k)
  int32_t kslice;  // hidden-size columns per slice
};

// Upper bound of slices for (B, m), independent of d: sizes the workspace.
int32_t router_max_slices(int32_t B, int32_t m);
RouterPlan router_plan(int dtype, int32_t B, int32_t d, int32_t m, const void* hidden,
                       const void* W1);

// Whether router stage 1 is small enough for its lean tiles to share the sweep's
// launch in a fused round (router_tile.h).  Stage 1 then keeps the MFMA tile whose
// sums the lean tile reproduces bit for bit, so a fused round and a separate
// route agree exactly; larger routers use the two-group form.
bool router_lean_tiles(const RouterPlan& plan, int32_t B, int32_t m);

hipError_t launch_router_stage1(const RouterPlan& plan, const void* hidden, const HiddenSel& sel,
                                int dtype, int32_t B, int32_t d, const void* W1, int32_t m,
                                float* zp, hipStream_t stream, ZeroFill zero = ZeroFill{nullptr, 0});

hipError_t launch_router_finish(const RouterPlan& plan, const HiddenSel& sel, int dtype,
                                const float* zp, int32_t B, int32_t m, const float* b1,
                                const void* W2, const float* b2, float tau, float* delta_al,
                                int32_t* choice, hipStream_t stream);

// Entropy policy: partials float4 {m, S, U, -} per (sequence, chunk), then one
// finish kernel.  Workspace: B * splits * 16 bytes.
SweepPlan entropy_plan(int32_t B, int32_t V);
hipError_t launch_entropy(const void* logits, int dtype, int64_t row_stride, int32_t total_rows,
                          int32_t V, int32_t B, const int32_t* row0, int32_t rows_per_seq,
                          const int32_t* pos, float tau, float* entropy, int32_t* choice,
                          void* workspace, hipStream_t stream);

// Lazy catch-up bookkeeping, one thread per sequence.
hipError_t launch_catchup(int32_t B, const int32_t* cur, const int32_t* accept_len,
                          const int32_t* nxt, int32_t* backlog, int32_t* switch_flag,
                          int32_t* catchup_len, hipStream_t stream);

struct RoutedArgs;
// Fused round: router finish + routed acceptance in one kernel per sequence.
// A fused round runs router stage 1 and the argmax sweep in one launch when the
// router takes the GEMV path for at most 8 sequences with 16-byte aligned
// operands; its sweep then uses few_rows_plan, whose chunk count lets the final
// kernel merge every row of a sequence (at most rows_per_seq rows) in one pass.
bool round_stage1_fused(const RouterPlan& plan, int hidden_dtype, const void* hidden, int32_t B,
                        int32_t d, const void* W1);
SweepPlan few_rows_plan(int32_t rows, int32_t V, int32_t rows_per_seq);
// Router stage 1 and the sweep: one launch if `fused`, else the two launches of
// launch_router_stage1 and launch_sweep.
hipError_t launch_round_stage1(bool fused, const RouterPlan& plan, int hidden_dtype,
                               const void* hidden, int32_t B, int32_t d, const void* W1, int32_t m,
                               float* zp, const void* logits, int logits_dtype, int64_t row_stride,
                               int32_t rows, int32_t V, SweepPlan sp, Partial* part,
                               hipStream_t stream);
hipError_t launch_round_chain_finalize(int hidden_dtype, const RouterPlan& plan, const float* zp,
                                       int32_t B, int32_t m, const float* b1, const void* W2,
                                       const float* b2, float tau, float* delta_al,
                                       int32_t* choice, const Partial* part, int32_t splits,
                                       int32_t K, const int32_t* draft, int32_t* accept_len,
                                       int32_t* bonus, int32_t* row_argmax, hipStream_t stream);
hipError_t launch_round_finalize(int hidden_dtype, const RouterPlan& plan, const float* zp, int32_t B,
                                 int32_t m, const float* b1, const void* W2, const float* b2,
                                 float tau, float* delta_al, int32_t* choice,
                                 const RoutedArgs& args, hipStream_t stream);

}  // namespace wf
