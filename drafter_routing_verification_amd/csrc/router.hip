// WhiFlash-Neural router (WhiFlash paper, section 3.3.2 and Appendix A):
//   dal[b] = W2 . GELU(W1 h_b + b1) + b2,  choice[b] = dal[b] > tau.
// Two first-stage kernels write fixed partial sums of the second layer,
// part[b * P + p] = sum over hidden units j of slice p of W2[j] * GELU(z[b, j]):
//   - router_gemv: small batches or float32.  One wave64 per hidden unit j
//     streams row j of W1 once with coalesced 16-byte loads and dots it with up
//     to 8 hidden states at a time; the dot is reduced across the wave with
//     shuffles, then GELU and the W2 product run in float32.  P = m.
//   - router_mfma: bf16 batches of 16 or more.  A workgroup computes a 32 (j) x
//     32 (b) tile of z with v_mfma_f32_16x16x32_bf16 (float32 accumulate), its
//     eight waves splitting the hidden size; GELU and W2 are applied to the
//     summed accumulators and each 16-unit slice of j yields one partial.
//     P = 2 * ceil(m / 32).
// router_reduce then sums the P partials of each sequence in a fixed order, so
// results are bitwise reproducible run to run, adds b2 and thresholds.
#include <math.h>

#include "common.h"

namespace wf {
namespace {

constexpr int kTileJ = 32;          // hidden units per MFMA workgroup tile
constexpr int kTileB = 32;          // sequences per MFMA workgroup tile
constexpr int kMfmaWaves = 8;       // waves splitting the hidden size of one tile
constexpr int kGemvUnroll = 4;      // 16-byte vectors in flight per lane in the GEMV

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_to_f32(unsigned short b) { return __uint_as_float(static_cast<unsigned>(b) << 16); }

template <int DT>
__device__ inline float load_elem(const void* p, int64_t i) {
  if constexpr (DT == WF_BF16) return bf16_to_f32(static_cast<const unsigned short*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

__device__ inline float gelu(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

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

// One wave per hidden unit j and NB sequences: row j of W1 is streamed once.
// VEC: rows are 16-byte aligned and d is a multiple of the vector width, so
// each lane reads 16-byte vectors, kGemvUnroll of them in flight.
template <int DT, int NB, bool VEC>
__global__ __launch_bounds__(kThreads) void router_gemv_kernel(
    const void* __restrict__ hidden, int B, int d, const void* __restrict__ W1,
    const float* __restrict__ b1, int m, const void* __restrict__ W2, float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int b0 = blockIdx.y * NB;
  if (j >= m) return;
  const int nb = min(NB, B - b0);
  float acc[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) acc[q] = 0.f;
  if constexpr (VEC) {
    constexpr int kPer = DT == WF_BF16 ? 8 : 4;
    const int nv = d / kPer;
    const u32x4* wr = reinterpret_cast<const u32x4*>(W1) + static_cast<int64_t>(j) * nv;
    const u32x4* hr = reinterpret_cast<const u32x4*>(hidden) + static_cast<int64_t>(b0) * nv;
    int v = lane;
    for (; v + (kGemvUnroll - 1) * 64 < nv; v += kGemvUnroll * 64) {
      u32x4 w[kGemvUnroll];
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u) w[u] = wr[v + u * 64];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        if (q < nb) {
          u32x4 h[kGemvUnroll];
#pragma unroll
          for (int u = 0; u < kGemvUnroll; ++u) h[u] = hr[static_cast<int64_t>(q) * nv + v + u * 64];
#pragma unroll
          for (int u = 0; u < kGemvUnroll; ++u) acc[q] = dot16<DT>(w[u], h[u], acc[q]);
        }
      }
    }
    for (; v < nv; v += 64) {
      const u32x4 w = wr[v];
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if (q < nb) acc[q] = dot16<DT>(w, hr[static_cast<int64_t>(q) * nv + v], acc[q]);
    }
  } else {
    const int64_t wrow = static_cast<int64_t>(j) * d;
    for (int k = lane; k < d; k += 64) {
      const float w = load_elem<DT>(W1, wrow + k);
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if (q < nb) acc[q] = fmaf(w, load_elem<DT>(hidden, static_cast<int64_t>(b0 + q) * d + k), acc[q]);
    }
  }
  const float bias = b1 ? b1[j] : 0.f;
  const float w2 = load_elem<DT>(W2, j);
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    float s = acc[q];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == q && q < nb) part[static_cast<int64_t>(b0 + q) * m + j] = w2 * gelu(s + bias);
  }
}

// 16 bytes (8 bf16) of row `r` at column k, or zeros outside the matrix.
__device__ inline bf16x8 frag(const unsigned short* base, int r, int rows, int d, int k) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < rows && k < d) v = *reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(r) * d + k);
  return __builtin_bit_cast(bf16x8, v);
}

// One workgroup per 32 (hidden units j) x 32 (sequences b) tile of z^T; its
// eight waves split the hidden size into interleaved 32-wide k steps, and
// their accumulators are summed in LDS in a fixed order.
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of
// the A tile and column (l % 16) of the B tile, 8 consecutive k values starting
// at 8 * (l / 16); the accumulator of lane l holds rows 4 * (l / 16) + i,
// i = 0..3, of column l % 16.
__global__ __launch_bounds__(kMfmaWaves * 64) void router_mfma_kernel(
    const unsigned short* __restrict__ hidden, int B, int d, const unsigned short* __restrict__ W1,
    const float* __restrict__ b1, int m, const unsigned short* __restrict__ W2, int P,
    float* __restrict__ part) {
  __shared__ float red[kMfmaWaves][16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j0 = blockIdx.x * kTileJ;
  const int bb0 = blockIdx.y * kTileB;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int steps = (d + 31) / 32;
  // All operands of up to kU of this wave's k steps are loaded before their
  // MFMAs, so a hidden size of up to kU * 8 * 32 costs one memory round trip.
  constexpr int kU = 10;
  for (int base = w; base < steps; base += kU * kMfmaWaves) {
    bf16x8 a0[kU], a1[kU], h0[kU], h1[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int k = (base + u * kMfmaWaves) * 32 + kq;  // frag() zero-fills k >= d
      a0[u] = frag(W1, j0 + r, m, d, k);
      a1[u] = frag(W1, j0 + 16 + r, m, d, k);
      h0[u] = frag(hidden, bb0 + r, B, d, k);
      h1[u] = frag(hidden, bb0 + 16 + r, B, d, k);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (base + u * kMfmaWaves < steps) {
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[u], h0[u], acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[u], h1[u], acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[u], h0[u], acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[u], h1[u], acc[1][1], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][a * 8 + c * 4 + i][lane] = acc[a][c][i];
  __syncthreads();
  // Waves 0..3 each finish one 16 (j) x 16 (b) accumulator: fixed-order sum over
  // the eight waves, GELU and W2, then the sum over its 16 hidden units.
  if (w < 4) {
    const int a = w >> 1, c = w & 1;
    float sacc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float z = 0.f;
#pragma unroll
      for (int ww = 0; ww < kMfmaWaves; ++ww) z += red[ww][a * 8 + c * 4 + i][lane];
      const int j = j0 + a * 16 + (lane >> 4) * 4 + i;
      if (j < m) sacc += bf16_to_f32(W2[j]) * gelu(z + (b1 ? b1[j] : 0.f));
    }
    sacc += __shfl_xor(sacc, 16);
    sacc += __shfl_xor(sacc, 32);
    const int b = bb0 + c * 16 + r;
    if (lane < 16 && b < B) part[static_cast<int64_t>(b) * P + blockIdx.x * 2 + a] = sacc;
  }
}

// One wave per sequence: fixed-order sum of its P partials, + b2, threshold.
__global__ __launch_bounds__(kThreads) void router_reduce_kernel(
    const float* __restrict__ part, int P, int B, const float* __restrict__ b2, float tau,
    float* __restrict__ delta_al, int32_t* __restrict__ choice) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (b >= B) return;
  const float* p = part + static_cast<int64_t>(b) * P;
  float s = 0.f;
  for (int i = lane; i < P; i += 64) s += p[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) {
    const float v = s + (b2 ? *b2 : 0.f);
    delta_al[b] = v;
    choice[b] = v > tau ? 1 : 0;
  }
}

}  // namespace

bool router_use_mfma(int dtype, int32_t B, int32_t d, const void* hidden, const void* W1) {
  const bool aligned = (reinterpret_cast<uintptr_t>(hidden) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(W1) % 16 == 0) && (d % 8 == 0);
  return dtype == WF_BF16 && B >= 16 && aligned;
}

int32_t router_partials(int32_t B, int32_t m, bool mfma) {
  (void)B;
  return mfma ? 2 * ((m + kTileJ - 1) / kTileJ) : m;
}

template <int DT, int NB, bool VEC>
static void gemv_launch(dim3 grid, hipStream_t stream, const void* hidden, int32_t B, int32_t d,
                        const void* W1, const float* b1, int32_t m, const void* W2, float* part) {
  hipLaunchKernelGGL((router_gemv_kernel<DT, NB, VEC>), grid, dim3(kThreads), 0, stream, hidden, B,
                     d, W1, b1, m, W2, part);
}

template <int DT, bool VEC>
static void gemv_dispatch(const void* hidden, int32_t B, int32_t d, const void* W1, const float* b1,
                          int32_t m, const void* W2, float* part, hipStream_t stream) {
  const unsigned gx = (m + kWaves - 1) / kWaves;
  if (B == 1) gemv_launch<DT, 1, VEC>(dim3(gx, 1), stream, hidden, B, d, W1, b1, m, W2, part);
  else if (B <= 2) gemv_launch<DT, 2, VEC>(dim3(gx, 1), stream, hidden, B, d, W1, b1, m, W2, part);
  else if (B <= 4) gemv_launch<DT, 4, VEC>(dim3(gx, 1), stream, hidden, B, d, W1, b1, m, W2, part);
  else gemv_launch<DT, 8, VEC>(dim3(gx, (B + 7) / 8), stream, hidden, B, d, W1, b1, m, W2, part);
}

hipError_t launch_router_gemv(const void* hidden, int dtype, int32_t B, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, float* part,
                              hipStream_t stream) {
  const int per = dtype == WF_BF16 ? 8 : 4;
  const bool vec = (reinterpret_cast<uintptr_t>(hidden) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(W1) % 16 == 0) && (d % per == 0);
  if (dtype == WF_BF16) {
    if (vec) gemv_dispatch<WF_BF16, true>(hidden, B, d, W1, b1, m, W2, part, stream);
    else gemv_dispatch<WF_BF16, false>(hidden, B, d, W1, b1, m, W2, part, stream);
  } else {
    if (vec) gemv_dispatch<WF_F32, true>(hidden, B, d, W1, b1, m, W2, part, stream);
    else gemv_dispatch<WF_F32, false>(hidden, B, d, W1, b1, m, W2, part, stream);
  }
  return hipGetLastError();
}

hipError_t launch_router_mfma(const void* hidden, int32_t B, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, float* part,
                              hipStream_t stream) {
  const int tiles = (m + kTileJ - 1) / kTileJ;
  const int P = 2 * tiles;
  const dim3 grid(tiles, (B + kTileB - 1) / kTileB);
  hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(kMfmaWaves * 64), 0, stream,
                     static_cast<const unsigned short*>(hidden), B, d,
                     static_cast<const unsigned short*>(W1), b1, m,
                     static_cast<const unsigned short*>(W2), P, part);
  return hipGetLastError();
}

hipError_t launch_router_reduce(const float* part, int32_t P, int32_t B, const float* b2, float tau,
                                float* delta_al, int32_t* choice, hipStream_t stream) {
  hipLaunchKernelGGL(router_reduce_kernel, dim3((B + kWaves - 1) / kWaves), dim3(kThreads), 0,
                     stream, part, P, B, b2, tau, delta_al, choice);
  return hipGetLastError();
}

}  // namespace wf
