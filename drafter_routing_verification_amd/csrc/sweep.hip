// Full-vocabulary argmax sweep over target logits rows (greedy verification:
// the target's token at each drafted position is the lowest index holding the
// row maximum; WhiFlash paper, section 3.2, with greedy decoding).
//
// HBM-bound streaming kernel.  Each workgroup owns one chunk of one row and
// reads it once with 16-byte loads, 256 threads side by side so every wave64
// load instruction covers 1 KiB of contiguous memory.  A thread keeps its
// running maximum and the 16-byte vector where it first reached it (strict
// ">" in increasing index order keeps the earliest) together with that
// vector's data, and recovers the element index from it at the end.  The per-chunk
// (max, index) pair is reduced across the wave with cross-lane shuffles and
// across the four waves in LDS; ties go to the lower index at every level.
#include <math.h>

#include "common.h"
#include "elem.h"

namespace wf {
namespace {

constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// (v, i) beats (bv, bi) when larger, or equal with a lower index.
__device__ inline void take_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void argmax_sweep_kernel(
    const unsigned char* __restrict__ logits, int64_t row_bytes, int V, int splits,
    int chunk_vecs, int nvec, Partial* __restrict__ part) {
  using E = Elem<DT>;
  const int blk = blockIdx.x;
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
  int v = v0 + tid;
  for (; v + (kUnroll - 1) * kThreads < v1; v += kUnroll * kThreads) {
    u32x4 d[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) d[u] = load16(vp + v + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float m = E::vmax(d[u]);
      if (m > best) {
        best = m;
        bestv = v + u * kThreads;
        bestd = d[u];
      }
    }
  }
  for (; v < v1; v += kThreads) {
    const u32x4 d = load16(vp + v);
    const float m = E::vmax(d);
    if (m > best) {
      best = m;
      bestv = v;
      bestd = d;
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

#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(idx, off);
    take_better(best, idx, ov, oi);
  }
  __shared__ float sv[kWaves];
  __shared__ int si[kWaves];
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = idx;
  }
  __syncthreads();
  if (tid == 0) {
    float bv = sv[0];
    int bi = si[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) take_better(bv, bi, sv[w], si[w]);
    part[blk] = Partial{bv, bi};
  }
}

}  // namespace

SweepPlan sweep_plan(int32_t rows, int32_t V) {
  // Chunks of ~12.7K elements (~25 KB of bf16) per workgroup: many short
  // streams keep HBM busier than a few long ones (measured on the 4,992 x
  // 151,936 bf16 sweep: 12 chunks per row 215.8 us, 2 chunks 219.2 us, 24
  // chunks 244 us).  Small batches split further so a launch still has about
  // 2048 workgroups, but never below 2048 elements per chunk.
  constexpr int64_t kChunkTarget = 12800;
  constexpr int64_t kMinBlocks = 2048;
  constexpr int64_t kMinChunk = 2048;
  const int64_t max_splits = V / kMinChunk > 1 ? V / kMinChunk : 1;
  int64_t splits = (V + kChunkTarget - 1) / kChunkTarget;
  const int64_t for_blocks = (kMinBlocks + rows - 1) / (rows > 0 ? rows : 1);
  if (splits < for_blocks) splits = for_blocks;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  // Chunk starts on 256-element boundaries (512 B of bf16, 1 KiB of float32),
  // so no memory line is shared by two chunks of a row and fetched twice.
  int64_t chunk = (V + splits - 1) / splits;
  chunk = (chunk + 255) / 256 * 256;
  splits = (V + chunk - 1) / chunk;
  return SweepPlan{static_cast<int32_t>(splits), static_cast<int32_t>(chunk)};
}

hipError_t launch_sweep(const void* logits, int dtype, int64_t row_stride, int32_t rows, int32_t V,
                        SweepPlan plan, Partial* part, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(rows) * plan.splits;
  if (blocks == 0) return hipSuccess;
  const unsigned char* base = static_cast<const unsigned char*>(logits);
  if (dtype == WF_BF16) {
    using E = Elem<WF_BF16>;
    hipLaunchKernelGGL(argmax_sweep_kernel<WF_BF16>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, base, row_stride * E::kBytes, V, plan.splits,
                       plan.chunk / E::kPerVec, V / E::kPerVec, part);
  } else {
    using E = Elem<WF_F32>;
    hipLaunchKernelGGL(argmax_sweep_kernel<WF_F32>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, base, row_stride * E::kBytes, V, plan.splits,
                       plan.chunk / E::kPerVec, V / E::kPerVec, part);
  }
  return hipGetLastError();
}

}  // namespace wf
