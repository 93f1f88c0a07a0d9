// The router's first layer on the GEMV path (small batches or float32
// hidden states): one wave64 per hidden unit streams row j of W1 once and dots
// it with up to NB hidden states (WhiFlash paper, section 3.3.2 and Appendix A:
// z = W1 h + b1 before the GELU).  Shared by router_gemv_kernel and the
// small-batch round kernel that runs it beside the argmax sweep.
#pragma once

#include "common.h"
#include "elem.h"
#include "router_math.h"
#include "dpp.h"

namespace wf {

constexpr int kGemvUnroll = 4;  // 16-byte vectors in flight per lane in the GEMV

// Dot product of two 16-byte vectors, accumulated in float32.
template <int DT>
__device__ inline float dot16(u32x4 a, u32x4 b, float acc) {
  if constexpr (DT == WF_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = fmaf(__uint_as_float(a[q] << 16), __uint_as_float(b[q] << 16), acc);
      acc = fmaf(__uint_as_float(a[q] & 0xffff0000u), __uint_as_float(b[q] & 0xffff0000u), acc);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(a[q]), __uint_as_float(b[q]), acc);
  }
  return acc;
}

// One wave per hidden unit j and NB sequences: row j of W1 is streamed once;
// writes zp[b][j] = W1[j] . h_b.
// VEC: rows are 16-byte aligned and d is a multiple of the vector width, so
// each lane reads 16-byte vectors, kGemvUnroll of them in flight.
// Workgroup (bx, by) covers hidden units bx * 4 .. bx * 4 + 3 (one per wave) and
// sequences by * NB .. by * NB + NB - 1.  Uses no barrier.
template <int DT, int NB, bool VEC>
__device__ inline void gemv_tile(int bx, int by, const void* __restrict__ hidden, const HiddenSel& sel,
                                 int B, int d, const void* __restrict__ W1, int m,
                                 float* __restrict__ zp) {
  const int lane = threadIdx.x & 63;
  const int j = bx * kWaves + (threadIdx.x >> 6);
  const int b0 = by * NB;
  if (j >= m) return;
  const int nb = min(NB, B - b0);
  // Hidden row of each of this wave's sequences (-1: no valid row, dot stays 0).
  int64_t hrow[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) hrow[q] = q < nb ? hidden_row(sel, b0 + q) : -1;
  float acc[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) acc[q] = 0.f;
  if constexpr (VEC) {
    constexpr int kPer = DT == WF_BF16 ? 8 : 4;
    const int nv = d / kPer;
    const u32x4* wr = reinterpret_cast<const u32x4*>(W1) + static_cast<int64_t>(j) * nv;
    const u32x4* hb = reinterpret_cast<const u32x4*>(hidden);
    int v = lane;
    for (; v + (kGemvUnroll - 1) * 64 < nv; v += kGemvUnroll * 64) {
      u32x4 w[kGemvUnroll];
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u) w[u] = wr[v + u * 64];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        if (hrow[q] >= 0) {
          const u32x4* hr = hb + hrow[q] * nv;
          u32x4 h[kGemvUnroll];
#pragma unroll
          for (int u = 0; u < kGemvUnroll; ++u) h[u] = hr[v + u * 64];
#pragma unroll
          for (int u = 0; u < kGemvUnroll; ++u) acc[q] = dot16<DT>(w[u], h[u], acc[q]);
        }
      }
    }
    for (; v < nv; v += 64) {
      const u32x4 w = wr[v];
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if (hrow[q] >= 0) acc[q] = dot16<DT>(w, hb[hrow[q] * nv + v], acc[q]);
    }
  } else {
    const int64_t wrow = static_cast<int64_t>(j) * d;
    for (int k = lane; k < d; k += 64) {
      const float w = load_elem<DT>(W1, wrow + k);
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if (hrow[q] >= 0) acc[q] = fmaf(w, load_elem<DT>(hidden, hrow[q] * d + k), acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const float s = wave_sum_to_lane63(acc[q]);
    if (lane == 63 && q < nb) zp[static_cast<int64_t>(b0 + q) * m + j] = s;
  }
}

}  // namespace wf
