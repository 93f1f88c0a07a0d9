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

// Partial result of the argmax sweep over one chunk of one row: the chunk's
// maximum and the lowest index holding it.
struct Partial {
  float val;
  int32_t idx;
};

// How the sweep cuts rows into chunks.  `chunk` is a multiple of 8 elements so
// every chunk starts on a 16-byte boundary for both element types.
struct SweepPlan {
  int32_t splits;  // chunks per row
  int32_t chunk;   // elements per chunk (last chunk of a row may be shorter)
};

SweepPlan sweep_plan(int32_t rows, int32_t V);

hipError_t launch_sweep(const void* logits, int dtype, int64_t row_stride, int32_t rows, int32_t V,
                        SweepPlan plan, Partial* part, hipStream_t stream);

hipError_t launch_finalize_chain(const Partial* part, int32_t splits, int32_t B, int32_t K,
                                 const int32_t* draft, int32_t* accept_len, int32_t* bonus,
                                 int32_t* row_argmax, hipStream_t stream);

hipError_t launch_finalize_tree(const Partial* part, int32_t splits, int32_t B, int32_t N, int32_t V,
                                const int32_t* parent, const int32_t* draft_ids, const int32_t* d2t,
                                int32_t Vd, int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                                int32_t* row_argmax, hipStream_t stream);

hipError_t launch_finalize_routed(const Partial* part, int32_t splits, int32_t B, int32_t V,
                                  const int32_t* row_offsets, int32_t total_rows,
                                  const int32_t* choice, int32_t K, const int32_t* chain_draft,
                                  int32_t N, const int32_t* parent, const int32_t* draft_ids,
                                  const int32_t* d2t, int32_t Vd, int32_t* accept_len,
                                  int32_t* bonus, int32_t* best_node, int32_t* row_argmax,
                                  hipStream_t stream);

// Router: partial second-layer sums part[b * P + p] over P slices of the m
// hidden units, then a fixed-order reduction to delta_al and the threshold.
int32_t router_partials(int32_t B, int32_t m, bool mfma);
bool router_use_mfma(int dtype, int32_t B, int32_t d, const void* hidden, const void* W1);

hipError_t launch_router_gemv(const void* hidden, int dtype, int32_t B, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, float* part,
                              hipStream_t stream);

hipError_t launch_router_mfma(const void* hidden, int32_t B, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, float* part,
                              hipStream_t stream);

hipError_t launch_router_reduce(const float* part, int32_t P, int32_t B, const float* b2, float tau,
                                float* delta_al, int32_t* choice, hipStream_t stream);

}  // namespace wf
