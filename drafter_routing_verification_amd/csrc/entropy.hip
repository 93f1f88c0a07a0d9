// WhiFlash-Entropy policy (WhiFlash paper, section 3.3.1): the entropy of the
// target's next-token distribution (softmax of one logits row) at each
// sequence's final accepted position, thresholded into a drafter choice.
//
// One streaming pass per selected row.  A workgroup owns one chunk of the row;
// each thread keeps, in base 2, m = running maximum, S = sum of 2^y and
// U = sum of y 2^y with y = (x - m) log2(e), rescaling both when m grows:
// moving to m' multiplies every 2^y by f = 2^d, d = (m - m') log2(e), and
// shifts every y by d, so S' = S f and U' = (U + d S) f.  Chunks merge the
// same way, and H = ln 2 (log2 S - U / S).  All merges run in a fixed order.
#include <math.h>

#include "common.h"
#include "elem.h"
#include "ent_math.h"

namespace wf {
namespace {

constexpr int kEntUnroll = 8;  // 16-byte loads in flight per thread

template <int DT>
__global__ __launch_bounds__(kThreads) void entropy_partial_kernel(
    const unsigned char* __restrict__ logits, int64_t row_bytes, int total_rows, int V,
    const int32_t* __restrict__ row0, int rows_per_seq, const int32_t* __restrict__ pos,
    int splits, int chunk_vecs, int nvec, float4* __restrict__ part) {
  using E = Elem<DT>;
  const int blk = blockIdx.x;
  const int b = blk / splits;
  const int c = blk - b * splits;
  const int64_t row = select_row(row0, rows_per_seq, pos, total_rows, b);
  const int tid = threadIdx.x;
  Ent acc{-INFINITY, 0.f, 0.f};
  if (row >= 0) {
    const unsigned char* rowp = logits + row * row_bytes;
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp);
    const int v0 = c * chunk_vecs;
    const int v1 = min(v0 + chunk_vecs, nvec);
    auto absorb = [&](u32x4 d) {
      const float mv = E::vmax(d);
      if (mv > acc.m) ent_raise(acc, mv);
      const float mb = acc.m * kLog2e;
#pragma unroll
      for (int k = 0; k < E::kPerVec; ++k) ent_add(acc, E::at(d, k), mb);
    };
    // Each thread issues its whole batch of loads (missing ones masked off)
    // before absorbing any: one round trip per batch for the few workgroups
    // of this pass.
    for (int v = v0 + tid; v < v1; v += kEntUnroll * kThreads) {
      u32x4 d[kEntUnroll];
#pragma unroll
      for (int u = 0; u < kEntUnroll; ++u)
        if (v + u * kThreads < v1) d[u] = load16(vp + v + u * kThreads);
#pragma unroll
      for (int u = 0; u < kEntUnroll; ++u)
        if (v + u * kThreads < v1) absorb(d[u]);
    }
    if (c == splits - 1 && tid == 0) {
      for (int e = nvec * E::kPerVec; e < V; ++e) {
        const float x = E::scalar(rowp, e);
        Ent one{x, 1.f, 0.f};
        ent_merge(acc, one);
      }
    }
  }
  wave_ent_to_lane63(acc);
  __shared__ Ent red[kWaves];
  if ((tid & 63) == 63) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    Ent t = red[0];
    for (int w = 1; w < kWaves; ++w) ent_merge(t, red[w]);
    part[blk] = make_float4(t.m, t.S, t.U, 0.f);
  }
}

// One wave per sequence: fixed-order merge of its chunks, H, threshold.
__global__ __launch_bounds__(kThreads) void entropy_finish_kernel(
    const float4* __restrict__ part, int splits, int B, const int32_t* __restrict__ row0,
    int rows_per_seq, const int32_t* __restrict__ pos, int total_rows, float tau,
    float* __restrict__ entropy, int32_t* __restrict__ choice) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (b >= B) return;
  Ent acc{-INFINITY, 0.f, 0.f};
  for (int s = lane; s < splits; s += 64) {
    const float4 p = part[static_cast<int64_t>(b) * splits + s];
    ent_merge(acc, Ent{p.x, p.y, p.z});
  }
  wave_ent_to_lane63(acc);
  if (lane == 63) {
    const bool valid = select_row(row0, rows_per_seq, pos, total_rows, b) >= 0 && acc.S > 0.f;
    const float H = valid ? ent_value(acc) : NAN;
    entropy[b] = H;
    choice[b] = (valid && H > tau) ? 1 : 0;
  }
}

}  // namespace

SweepPlan entropy_plan(int32_t B, int32_t V) {
  // ~2048 workgroups over the B selected rows, chunks of at least 2048 elements.
  constexpr int64_t kTargetBlocks = 2048;
  constexpr int64_t kMinChunk = 2048;
  const int64_t max_splits = V / kMinChunk > 1 ? V / kMinChunk : 1;
  int64_t splits = (kTargetBlocks + B - 1) / (B > 0 ? B : 1);
  if (splits < 1) splits = 1;
  if (splits > max_splits) splits = max_splits;
  int64_t chunk = (V + splits - 1) / splits;
  chunk = (chunk + 7) / 8 * 8;
  splits = (V + chunk - 1) / chunk;
  return SweepPlan{static_cast<int32_t>(splits), static_cast<int32_t>(chunk)};
}

hipError_t launch_entropy(const void* logits, int dtype, int64_t row_stride, int32_t total_rows,
                          int32_t V, int32_t B, const int32_t* row0, int32_t rows_per_seq,
                          const int32_t* pos, float tau, float* entropy, int32_t* choice,
                          void* workspace, hipStream_t stream) {
  const SweepPlan plan = entropy_plan(B, V);
  float4* part = static_cast<float4*>(workspace);
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(B) * plan.splits);
  const unsigned char* base = static_cast<const unsigned char*>(logits);
  if (dtype == WF_BF16) {
    using E = Elem<WF_BF16>;
    hipLaunchKernelGGL(entropy_partial_kernel<WF_BF16>, dim3(blocks), dim3(kThreads), 0, stream,
                       base, row_stride * E::kBytes, total_rows, V, row0, rows_per_seq, pos,
                       plan.splits, plan.chunk / E::kPerVec, V / E::kPerVec, part);
  } else {
    using E = Elem<WF_F32>;
    hipLaunchKernelGGL(entropy_partial_kernel<WF_F32>, dim3(blocks), dim3(kThreads), 0, stream,
                       base, row_stride * E::kBytes, total_rows, V, row0, rows_per_seq, pos,
                       plan.splits, plan.chunk / E::kPerVec, V / E::kPerVec, part);
  }
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(entropy_finish_kernel, dim3((B + kWaves - 1) / kWaves), dim3(kThreads), 0,
                     stream, part, plan.splits, B, row0, rows_per_seq, pos, total_rows, tau, entropy,
                     choice);
  return hipGetLastError();
}

}  // namespace wf
