// The argmax sweep over one chunk of one logits row (greedy verification:
// the target's token at each drafted position is the lowest index holding the
// row maximum; WhiFlash paper, section 3.2, with greedy decoding), run by one
// workgroup.  Shared by the sweep kernel and the fused round kernel.
//
// HBM-bound streaming.  The threads read the chunk side by side with
// 16-byte non-temporal loads, so every wave64 load instruction covers 1 KiB of
// contiguous memory.  A thread keeps its running maximum, the 16-byte vector
// where it first reached it (strict ">" in increasing index order keeps the
// earliest) and that vector's data, and recovers the element index from it at
// the end.  The chunk's (max, index) pair is reduced across the wave with DPP
// lane moves and across the waves in LDS; ties go to the lower index at every
// level.
#pragma once

#include <math.h>

#include "common.h"
#include "elem.h"
#include "dpp.h"

namespace wf {

constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// In a large launch (every resident slot streaming, one load at a time per
// thread), the workgroups dispatched first and the last ones of every XCD issue
// their whole batch of loads at once instead: the first kSweepHeadBatch of the
// grid, while the slots fill, and the last kSweepTailBatch that each XCD takes
// (workgroup i goes to XCD i % 8), while they drain.  Each then has five times
// the bytes in flight when few workgroups are.  Same box, two trials, back-to-back
// sweeps alone, 4,352 / 4,992 rows of 151,936 and 2,816 rows of 128,256 bf16:
// 181.1-181.3 / 217.2-217.9 / 101.8-102.0 us streaming everywhere; 179.0-179.2 /
// 215.2-215.7 / 99.9-100.0 us with 4,096 head and 512 tail workgroups per XCD
// (head 2,048-6,144 and tail 256-1,024 within 0.3 us of that; the head alone
// 179.6 / 216.2 / 100.4, the tail alone 180.2 / 216.4 / 101.4).
constexpr unsigned kSweepHeadBatch = 4096;
constexpr unsigned kSweepTailBatch = 512;
constexpr unsigned kSweepXcds = 8;  // accelerator complex dies of an MI355X
__device__ inline bool sweep_edge_block() {
  return blockIdx.x < kSweepHeadBatch || blockIdx.x + kSweepXcds * kSweepTailBatch >= gridDim.x;
}

// (v, i) beats (bv, bi) when larger, or equal with a lower index.
__device__ inline void take_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// The wave step of the chunk's reduction is wave_argmax_to_lane63 (dpp.h).  A
// thread's running maximum never holds NaN (a NaN vector maximum never beats
// it), so the pairs it combines are totally ordered.

// Returns the chunk's (max, index) in thread 0 (other threads: unspecified).
// NT threads per workgroup (a multiple of 64).  Two forms of the stream:
//   kBatchTail false: full batches of kUnroll loads, then the remainder one
//     load at a time.  Best when every resident workgroup streams (the full
//     sweep: 32 waves per CU each with a load in flight keep HBM busy).
//   kBatchTail true: every batch, the last partial one included, issues all
//     its loads before the first compare (missing loads masked off).  Best
//     when fewer workgroups stream at once (the early-exit schedule).
template <int DT, int NT = kThreads, bool kBatchTail = false>
__device__ inline Partial sweep_chunk(int blk, const unsigned char* __restrict__ logits,
                                      int64_t row_bytes, int V, int splits, int chunk_vecs, int nvec,
                                      Partial* __restrict__ part) {
  using E = Elem<DT>;
  constexpr int kW = NT / 64;
  const int row = blk / splits;
  const int c = blk - row * splits;
  const unsigned char* rowp = logits + static_cast<int64_t>(row) * row_bytes;
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp);
  const int tid = threadIdx.x;
  const int v0 = c * chunk_vecs;
  const int v1 = min(v0 + chunk_vecs, nvec);

  // The vector where `best` was first reached stays in registers, so the index
  // is recovered without a dependent re-load after the stream.
  float best = -INFINITY;
  int bestv = -1;
  u32x4 bestd = {0u, 0u, 0u, 0u};
  if constexpr (kBatchTail) {
    for (int v = v0 + tid; v < v1; v += kUnroll * NT) {
      u32x4 d[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (v + u * NT < v1) d[u] = load16(vp + v + u * NT);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (v + u * NT < v1) {
          const float m = E::vmax(d[u]);
          if (m > best) {
            best = m;
            bestv = v + u * NT;
            bestd = d[u];
          }
        }
      }
    }
  } else {
    int v = v0 + tid;
    for (; v + (kUnroll - 1) * NT < v1; v += kUnroll * NT) {
      u32x4 d[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) d[u] = load16(vp + v + u * NT);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float m = E::vmax(d[u]);
        if (m > best) {
          best = m;
          bestv = v + u * NT;
          bestd = d[u];
        }
      }
    }
    for (; v < v1; v += NT) {
      const u32x4 d = load16(vp + v);
      const float m = E::vmax(d);
      if (m > best) {
        best = m;
        bestv = v;
        bestd = d;
      }
    }
  }

  int idx = INT_MAX;
  if (v0 + tid < v1) {
    // No element above -inf (all -inf, or NaN): the thread's first element is
    // the first occurrence of -inf, and a valid index in every case.
    idx = bestv >= 0 ? bestv * E::kPerVec + E::first_equal(bestd, best) : (v0 + tid) * E::kPerVec;
  } else {
    best = -INFINITY;
  }
  // Elements past the last full vector (V not a multiple of the vector width).
  if (c == splits - 1 && tid == 0) {
    for (int e = nvec * E::kPerVec; e < V; ++e) {
      const float x = E::scalar(rowp, e);
      if (x > best || idx == INT_MAX) {
        best = x;
        idx = e;
      }
    }
  }

  __shared__ float sv[kW];
  __shared__ int si[kW];
  const int lane = tid & 63, wave = tid >> 6;
  // DPP lane moves instead of cross-lane shuffles: each shuffle step was two
  // ds_bpermute round trips and a branchy compare.  Same box, sweep kernel
  // alone, two interleaved trials: 32 chains 27.1-27.2 -> 26.4-26.6 us, 8 trees
  // 24.3-24.5 -> 24.1 us, 256 chains 186.0-186.3 -> 184.9-186.0 us,
  // Llama-shape chains 110.1-110.3 -> 103.5 us.
  wave_argmax_to_lane63(best, idx);
  if (lane == 63) {
    sv[wave] = best;
    si[wave] = idx;
  }
  __syncthreads();
  if (tid == 0) {
    float bv = sv[0];
    int bi = si[0];
#pragma unroll
    for (int w = 1; w < kW; ++w) take_better(bv, bi, sv[w], si[w]);
    part[blk] = Partial{bv, bi};
    return Partial{bv, bi};
  }
  return Partial{best, idx};
}

}  // namespace wf
