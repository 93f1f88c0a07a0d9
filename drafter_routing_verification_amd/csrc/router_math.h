// Router arithmetic shared by the router kernels and the fused round kernel:
// element loads, exact-erf GELU, and the per-sequence finish (WhiFlash paper,
// section 3.3.2 and Appendix A): z = sum of the slice partials + b1, then
// dal = W2 . GELU(z) + b2, in float32 and a fixed order.
#pragma once

#include <math.h>

#include "common.h"
#include "dpp.h"

namespace wf {

__device__ inline float bf16_to_f32(unsigned short b) { return __uint_as_float(static_cast<unsigned>(b) << 16); }

template <int DT>
__device__ inline float load_elem(const void* p, int64_t i) {
  if constexpr (DT == WF_BF16) return bf16_to_f32(static_cast<const unsigned short*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

__device__ inline float gelu(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Each thread owns up to kFinishPer hidden units per pass of the finish; all
// their partials, biases and W2 entries are loaded before any is used, so a
// pass costs one memory round trip.
constexpr int kFinishPer = 4;

// Loads of the first pass of the finish of sequence b (hidden units
// j = threadIdx.x + u * 256, u < kFinishPer), issued before any is used.
struct FinishIn {
  float part[kMaxRouterSlices][kFinishPer];
  float bias[kFinishPer], w2[kFinishPer];
  float b2v;     // the second-layer bias (first pass only)
  bool has_row;  // the sequence has a hidden row (first pass only)
};

// The first pass (base == 0) also loads b2 and the sequence's hidden-row
// selection, so no load is left for after the reduction.
template <int DT>
__device__ inline void finish_load_pass(FinishIn& in, const float* __restrict__ zp, int KS, int B,
                                        int m, int b, int base, const float* __restrict__ b1,
                                        const void* __restrict__ W2, const float* __restrict__ b2,
                                        const HiddenSel& sel) {
  if (base == 0) {
    in.b2v = b2 ? *b2 : 0.f;
    in.has_row = hidden_row(sel, b) >= 0;
  }
  const int64_t slice_stride = static_cast<int64_t>(B) * m;
  const float* zb = zp + static_cast<int64_t>(b) * m;
  // Every load is issued unconditionally, from an index that is always valid
  // (unit m - 1, slice KS - 1); finish_fold_pass drops what lies past m or KS.
  // Guarded loads let the compiler sink each first use into the load's own
  // branch, so every step of this loop waited for its load: four round trips
  // instead of one.
#pragma unroll
  for (int u = 0; u < kFinishPer; ++u) {
    const int j = base + u * kThreads + threadIdx.x;
    const int jc = j < m ? j : m - 1;
#pragma unroll
    for (int s = 0; s < kMaxRouterSlices; ++s)
      in.part[s][u] = zb[(s < KS ? s : KS - 1) * slice_stride + jc];
    in.bias[u] = b1 ? b1[jc] : 0.f;
    in.w2[u] = load_elem<DT>(W2, jc);
  }
}

// Units past m (their loads repeated unit m - 1) and slices past KS are
// dropped here, by selects on loaded values.
__device__ inline float finish_fold_pass(const FinishIn& in, int KS, int m, int base, float acc) {
#pragma unroll
  for (int u = 0; u < kFinishPer; ++u) {
    float z = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxRouterSlices; ++s) z += s < KS ? in.part[s][u] : 0.f;
    const float c = in.w2[u] * gelu(z + in.bias[u]);
    acc += base + u * kThreads + static_cast<int>(threadIdx.x) < m ? c : 0.f;
  }
  return acc;
}

// Delta-AL of sequence b from zp[s][b][j] (s < KS), computed by the whole
// workgroup, given the first pass already loaded in `first`; `red` is LDS of
// kWaves floats.  Every thread returns the value; NaN when the sequence has
// no hidden row.
template <int DT>
__device__ inline float router_finish_compute(const FinishIn& first, const float* __restrict__ zp,
                                              const HiddenSel& sel, int KS, int B, int m, int b,
                                              const float* __restrict__ b1,
                                              const void* __restrict__ W2,
                                              const float* __restrict__ b2, float* red) {
  const int tid = threadIdx.x;
  float acc = finish_fold_pass(first, KS, m, 0, 0.f);
  for (int base = kThreads * kFinishPer; base < m; base += kThreads * kFinishPer) {
    FinishIn in;
    finish_load_pass<DT>(in, zp, KS, B, m, b, base, b1, W2, b2, sel);
    acc = finish_fold_pass(in, KS, m, base, acc);
  }
  acc = wave_sum_to_lane63(acc);
  __syncthreads();  // red may still be in use by the caller
  if ((tid & 63) == 63) red[tid >> 6] = acc;
  __syncthreads();
  float v = red[0];
  for (int w = 1; w < kWaves; ++w) v += red[w];
  v += first.b2v;
  if (!first.has_row) v = NAN;  // no hidden row for this sequence
  return v;
}

template <int DT>
__device__ inline float router_finish_sequence(const float* __restrict__ zp, const HiddenSel& sel,
                                               int KS, int B, int m, int b,
                                               const float* __restrict__ b1,
                                               const void* __restrict__ W2,
                                               const float* __restrict__ b2, float* red) {
  FinishIn first;
  finish_load_pass<DT>(first, zp, KS, B, m, b, 0, b1, W2, b2, sel);
  return router_finish_compute<DT>(first, zp, sel, KS, B, m, b, b1, W2, b2, red);
}

}  // namespace wf
