// Router arithmetic shared by the router kernels and the fused round kernel:
// element loads, exact-erf GELU, and the per-sequence finish (WhiFlash paper,
// section 3.3.2 and Appendix A): z = sum of the slice partials + b1, then
// dal = W2 . GELU(z) + b2, in float32 and a fixed order.
#pragma once

#include <math.h>

#include "common.h"

namespace wf {

__device__ inline float bf16_to_f32(unsigned short b) { return __uint_as_float(static_cast<unsigned>(b) << 16); }

template <int DT>
__device__ inline float load_elem(const void* p, int64_t i) {
  if constexpr (DT == WF_BF16) return bf16_to_f32(static_cast<const unsigned short*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

__device__ inline float gelu(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Each thread owns up to kFinishPer hidden units per pass; all their partials,
// biases and W2 entries are loaded before any is used, so a pass costs one
// memory round trip.
constexpr int kFinishPer = 4;

// Delta-AL of sequence b from zp[s][b][j] (s < KS), computed by the whole
// workgroup; `red` is LDS of kWaves floats.  Every thread returns the value;
// NaN when the sequence has no hidden row.
template <int DT>
__device__ inline float router_finish_sequence(const float* __restrict__ zp, const HiddenSel& sel,
                                               int KS, int B, int m, int b,
                                               const float* __restrict__ b1,
                                               const void* __restrict__ W2,
                                               const float* __restrict__ b2, float* red) {
  const int tid = threadIdx.x;
  const int64_t slice_stride = static_cast<int64_t>(B) * m;
  const float* zb = zp + static_cast<int64_t>(b) * m;
  float acc = 0.f;
  for (int base = 0; base < m; base += kThreads * kFinishPer) {
    float part[kMaxRouterSlices][kFinishPer];
    float bias[kFinishPer], w2[kFinishPer];
#pragma unroll
    for (int u = 0; u < kFinishPer; ++u) {
      const int j = base + u * kThreads + tid;
      const bool ok = j < m;
#pragma unroll
      for (int s = 0; s < kMaxRouterSlices; ++s)
        part[s][u] = (ok && s < KS) ? zb[s * slice_stride + j] : 0.f;
      bias[u] = (ok && b1) ? b1[j] : 0.f;
      w2[u] = ok ? load_elem<DT>(W2, j) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kFinishPer; ++u) {
      if (base + u * kThreads + tid < m) {
        float z = 0.f;
#pragma unroll
        for (int s = 0; s < kMaxRouterSlices; ++s)
          if (s < KS) z += part[s][u];
        acc += w2[u] * gelu(z + bias[u]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  __syncthreads();  // red may still be in use by the caller
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  float v = red[0];
  for (int w = 1; w < kWaves; ++w) v += red[w];
  v += b2 ? *b2 : 0.f;
  if (hidden_row(sel, b) < 0) v = NAN;  // no hidden row for this sequence
  return v;
}

}  // namespace wf
