// Full-vocabulary argmax sweep kernel: one workgroup per chunk of a row
// (the per-chunk work is in sweep_body.h).
#include "common.h"
#include "sweep_body.h"
#include "dpp.h"

#ifndef WF_SWEEP_THREADS
#define WF_SWEEP_THREADS 256
#endif
#ifndef WF_SWEEP_CHUNK
#define WF_SWEEP_CHUNK 10000
#endif

namespace wf {
namespace {

constexpr int kSweepThreads = WF_SWEEP_THREADS;

// Workgroups are handed to the 8 XCDs round robin (workgroup i to XCD i % 8).
// Renumber them so that XCD x sweeps one contiguous range of chunks, in order:
// the n chunks are cut into 8 ranges of n / 8 (the first n % 8 one longer).
__device__ inline int xcd_contiguous_block() {
  const unsigned n = gridDim.x, q = n / kSweepXcds, r = n % kSweepXcds;
  const unsigned x = blockIdx.x % kSweepXcds, k = blockIdx.x / kSweepXcds;
  return static_cast<int>(x * q + (x < r ? x : r) + k);
}

// Launches of at most kSmallLaunch workgroups fit in about four rounds of the
// 2,048 resident slots (256 CUs x 8 workgroups of 4 waves).  There each thread
// issues its whole batch of loads before comparing (sweep_chunk's kBatchTail
// form); larger launches keep every slot busy with one load at a time per
// thread.  Same-box A/B, sweep kernel alone, two interleaved trials: with the
// switch at 8,192 instead of 4,096, 32 chains (544 rows, 5,984 workgroups)
// 29.3-29.4 -> 27.2 us and 8 trees (488 rows, 5,368 workgroups) 26.3-26.5 ->
// 24.4 us; 16,384 gave the same.  Batching the Llama-shape launch (25,344
// workgroups) changed nothing (104.7-104.9 against 104.9 us), and the
// 47,872- and 54,912-workgroup launches slowed by 4 us (190.7 -> 194.7-195.2,
// 210.7-211.0 -> 215.5-216.0).
#ifndef WF_SWEEP_SMALL_LAUNCH
#define WF_SWEEP_SMALL_LAUNCH 8192
#endif
constexpr int64_t kSmallLaunch = WF_SWEEP_SMALL_LAUNCH;

template <int DT, bool kBatch>
__global__ __launch_bounds__(kSweepThreads) void argmax_sweep_kernel(
    const unsigned char* __restrict__ logits, int64_t row_bytes, int V, int splits,
    int chunk_vecs, int nvec, Partial* __restrict__ part) {
  if (kBatch || sweep_edge_block())
    sweep_chunk<DT, kSweepThreads, true>(xcd_contiguous_block(), logits, row_bytes, V, splits,
                                         chunk_vecs, nvec, part);
  else
    sweep_chunk<DT, kSweepThreads, false>(xcd_contiguous_block(), logits, row_bytes, V, splits,
                                          chunk_vecs, nvec, part);
}

// The sweep's reads without its comparisons: the same chunks, workgroups,
// numbering and loads, each thread folding its data into an XOR.  Workgroup
// 0's XOR (chunk 0 of row 0) is written to *sink so the loads stay live.
template <bool kBatch>
__global__ __launch_bounds__(kSweepThreads) void stream_read_kernel(
    const unsigned char* __restrict__ logits, int64_t row_bytes, int splits, int chunk_vecs,
    int nvec, unsigned* __restrict__ sink) {
  const int blk = xcd_contiguous_block();
  const int row = blk / splits;
  const int c = blk - row * splits;
  const u32x4* vp = reinterpret_cast<const u32x4*>(logits + static_cast<int64_t>(row) * row_bytes);
  const int v0 = c * chunk_vecs;
  const int v1 = min(v0 + chunk_vecs, nvec);
  unsigned acc = 0;
  int v = v0 + threadIdx.x;
  if (kBatch || sweep_edge_block()) {
    for (; v < v1; v += kUnroll * kSweepThreads) {
      u32x4 d[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (v + u * kSweepThreads < v1) d[u] = load16(vp + v + u * kSweepThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (v + u * kSweepThreads < v1) acc ^= d[u][0] ^ d[u][1] ^ d[u][2] ^ d[u][3];
    }
  } else {
    for (; v + (kUnroll - 1) * kSweepThreads < v1; v += kUnroll * kSweepThreads) {
      u32x4 d[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) d[u] = load16(vp + v + u * kSweepThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= d[u][0] ^ d[u][1] ^ d[u][2] ^ d[u][3];
    }
    for (; v < v1; v += kSweepThreads) {
      const u32x4 d = load16(vp + v);
      acc ^= d[0] ^ d[1] ^ d[2] ^ d[3];
    }
  }
  __shared__ unsigned sx[kSweepThreads / 64];
  acc = wave_xor_to_lane63(acc);  // the same DPP reduction shape as the sweep's
  if ((threadIdx.x & 63) == 63) sx[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (blk == 0 && threadIdx.x == 0) {
    unsigned t = 0;
    for (int w = 0; w < kSweepThreads / 64; ++w) t ^= sx[w];
    *sink = t;
  }
}

}  // namespace

bool sweep_batched(int64_t blocks) { return blocks <= kSmallLaunch; }

SweepPlan sweep_plan(int32_t rows, int32_t V) {
  // 256-thread workgroups over chunks of ~10K elements (~20 KB of bf16),
  // rounded down to an odd count per row: 15 per 151,936-wide row (10,240
  // elements: 5 loads of 16 bytes per thread) and 13 per 128,256-wide row.
  // Small batches split further so a launch still has about 2048 workgroups,
  // but never below 2048 elements per chunk.
  //
  // Same box, bench line on the 256-chain and routed workloads, two interleaved
  // trials each, sweep kernel alone (whole step):
  //   11 chunks per row (13,824)  184.2-184.3 us (199.9-200.3)   routed 209.3 (223.4-223.5)
  //   13 chunks (11,776)          183.3-183.4 us (198.9-199.1)   routed 208.3-208.7 (221.9-222.3)
  //   15 chunks (10,240)          182.2 us (198.1-198.3)         routed 207.7-207.9 (221.0-221.3)
  //   17 chunks (9,216)           187.7-188.0 us (203.9-204.0)   routed 213.7 (228.0-228.1)
  //   19 chunks (8,192)           192.6-192.8 us (208.7-208.9)   routed 216.7-216.8 (232.1-232.4)
  // The same change moved the 32-chain and 8-tree sweeps by -0.2 us, the
  // Llama-shape sweep (9 -> 13 chunks) within its spread, the one-sequence round
  // not at all.  Earlier, with the XCD-contiguous numbering and the 12.8K-14.4K
  // targets:
  //
  // Same-box A/B on the Llama-shape chain workload (2,816 x 128,256 rows, three
  // interleaved trials): 9 chunks per row (this target) 104.96-105.31 us for
  // the sweep, 11 chunks (a 12.8K target) 105.83-106.37 us.  The 151,936-wide
  // rows get 11 chunks either way.
  //
  // Same-process A/B, whole verify call, on the routed / chain / Llama-shape
  // chain workloads (4,992 x 151,936, 4,352 x 151,936 and 2,816 x 128,256
  // rows; median of 5 interleaved trials):
  //   11 chunks per row, XCD-contiguous numbering   219.0 / 187.7 / 107.5 us
  //   11 chunks per row, launch order               219.9 / 189.5 / 106.8 us
  //   12 per 151,936-wide row (the earlier rule)    223.6 / 191.6 / 106.7 us
  //   12, XCD-contiguous numbering                  222.6 / 189.7 / 107.4 us
  //   13 chunks                                     222.1 / 189.7 / 107.4 us
  //   10 chunks                                     225.5 / 195.1 / 108.8 us
  // Chunks of 8K-11K or of 16K elements were slower still.  Before that
  // (routed / chain workloads, 12 chunks per row at 219.0 / 191.8 us): 512
  // threads over 30,720-element chunks 246.8 / 215.9 us, or 223.4 / 197.3 us
  // with every load batch issued whole; 256 threads with whole batches 228.6 /
  // 197.6 us; 2 chunks per row 219.2 us and 24 chunks 244 us (routed).
  constexpr int64_t kChunkTarget = WF_SWEEP_CHUNK;
  constexpr int64_t kMinBlocks = 2048 * 256 / kSweepThreads;
  constexpr int64_t kMinChunk = 2048;
  const int64_t max_splits = V / kMinChunk > 1 ? V / kMinChunk : 1;
  int64_t splits = (V + kChunkTarget - 1) / kChunkTarget;
  // An odd number of chunks per row measured faster than its even neighbours.
  if (splits > 2 && splits % 2 == 0) --splits;
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
  const dim3 grid(static_cast<unsigned>(blocks)), block(kSweepThreads);
  const bool small = blocks <= kSmallLaunch;
  if (dtype == WF_BF16) {
    using E = Elem<WF_BF16>;
    const int64_t rb = row_stride * E::kBytes;
    const int cv = plan.chunk / E::kPerVec, nv = V / E::kPerVec;
    if (small)
      hipLaunchKernelGGL((argmax_sweep_kernel<WF_BF16, true>), grid, block, 0, stream, base, rb, V,
                         plan.splits, cv, nv, part);
    else
      hipLaunchKernelGGL((argmax_sweep_kernel<WF_BF16, false>), grid, block, 0, stream, base, rb, V,
                         plan.splits, cv, nv, part);
  } else {
    using E = Elem<WF_F32>;
    const int64_t rb = row_stride * E::kBytes;
    const int cv = plan.chunk / E::kPerVec, nv = V / E::kPerVec;
    if (small)
      hipLaunchKernelGGL((argmax_sweep_kernel<WF_F32, true>), grid, block, 0, stream, base, rb, V,
                         plan.splits, cv, nv, part);
    else
      hipLaunchKernelGGL((argmax_sweep_kernel<WF_F32, false>), grid, block, 0, stream, base, rb, V,
                         plan.splits, cv, nv, part);
  }
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* logits, int dtype, int64_t row_stride, int32_t rows,
                              int32_t V, SweepPlan plan, unsigned* sink, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(rows) * plan.splits;
  if (blocks == 0) return hipSuccess;
  const int per = dtype == WF_BF16 ? Elem<WF_BF16>::kPerVec : Elem<WF_F32>::kPerVec;
  const int64_t bytes = dtype == WF_BF16 ? Elem<WF_BF16>::kBytes : Elem<WF_F32>::kBytes;
  if (blocks <= kSmallLaunch)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kSweepThreads), 0, stream, static_cast<const unsigned char*>(logits),
                       row_stride * bytes, plan.splits, plan.chunk / per, V / per, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kSweepThreads), 0, stream, static_cast<const unsigned char*>(logits),
                       row_stride * bytes, plan.splits, plan.chunk / per, V / per, sink);
  return hipGetLastError();
}

}  // namespace wf
