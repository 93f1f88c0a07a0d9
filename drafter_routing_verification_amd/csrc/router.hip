// WhiFlash-Neural router (WhiFlash paper, section 3.3.2 and Appendix A):
//   dal[b] = W2 . GELU(W1 h_b + b1) + b2,  choice[b] = dal[b] > tau.
// Two first-stage kernels write fixed partial sums of the second layer,
// part[b * P + p] = sum over hidden units j of slice p of W2[j] * GELU(z[b, j]):
//   - router_gemv: small batches or float32.  One wave64 per hidden unit j
//     streams row j of W1 once with coalesced loads and dots it with up to
//     kGemvBatch hidden states at a time; the dot is reduced across the wave
//     with shuffles, then GELU and the W2 product run in float32.  P = m.
//   - router_mfma: bf16 batches of 16 or more.  Each wave computes a 32 (j) x
//     32 (b) tile of z with v_mfma_f32_16x16x32_bf16 (float32 accumulate) over
//     the whole hidden size and applies GELU and W2 to its accumulators before
//     reducing over its 32 hidden units.  P = ceil(m / 32).
// router_reduce then sums the P partials of each sequence in a fixed order, so
// results are bitwise reproducible run to run, adds b2 and thresholds.
#include <math.h>

#include "common.h"

namespace wf {
namespace {

constexpr int kGemvBatch = 8;
constexpr int kTileJ = 32;
constexpr int kTileB = 32;

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

// One wave per hidden unit j, kGemvBatch sequences per grid row.
template <int DT>
__global__ __launch_bounds__(kThreads) void router_gemv_kernel(
    const void* __restrict__ hidden, int B, int d, const void* __restrict__ W1,
    const float* __restrict__ b1, int m, const void* __restrict__ W2, float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int b0 = blockIdx.y * kGemvBatch;
  if (j >= m) return;
  const int nb = min(kGemvBatch, B - b0);
  float acc[kGemvBatch];
#pragma unroll
  for (int q = 0; q < kGemvBatch; ++q) acc[q] = 0.f;
  const int64_t wrow = static_cast<int64_t>(j) * d;
  for (int k = lane; k < d; k += 64) {
    const float w = load_elem<DT>(W1, wrow + k);
#pragma unroll
    for (int q = 0; q < kGemvBatch; ++q)
      if (q < nb) acc[q] = fmaf(w, load_elem<DT>(hidden, static_cast<int64_t>(b0 + q) * d + k), acc[q]);
  }
  const float bias = b1 ? b1[j] : 0.f;
  const float w2 = load_elem<DT>(W2, j);
#pragma unroll
  for (int q = 0; q < kGemvBatch; ++q) {
    float s = acc[q];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == q && q < nb) part[static_cast<int64_t>(b0 + q) * m + j] = w2 * gelu(s + bias);
  }
}

// 16 bytes (8 bf16) of row `r` at column k, or zeros when the row is out of range.
__device__ inline bf16x8 frag(const unsigned short* base, int r, int rows, int d, int k) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < rows && k < d) v = *reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(r) * d + k);
  return __builtin_bit_cast(bf16x8, v);
}

// One wave per 32 x 32 tile of z^T (rows: hidden units j, columns: sequences b).
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of
// the A tile and column (l % 16) of the B tile, 8 consecutive k values starting
// at 8 * (l / 16); the accumulator of lane l holds rows 4 * (l / 16) + i,
// i = 0..3, of column l % 16.
__global__ __launch_bounds__(64) void router_mfma_kernel(
    const unsigned short* __restrict__ hidden, int B, int d, const unsigned short* __restrict__ W1,
    const float* __restrict__ b1, int m, const unsigned short* __restrict__ W2, int P,
    float* __restrict__ part) {
  const int lane = threadIdx.x;
  const int j0 = blockIdx.x * kTileJ;
  const int bb0 = blockIdx.y * kTileB;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < d; k0 += 32) {
    const int k = k0 + kq;
    const bf16x8 a0 = frag(W1, j0 + r, m, d, k);
    const bf16x8 a1 = frag(W1, j0 + 16 + r, m, d, k);
    const bf16x8 h0 = frag(hidden, bb0 + r, B, d, k);
    const bf16x8 h1 = frag(hidden, bb0 + 16 + r, B, d, k);
    acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, h0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, h1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, h0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, h1, acc[1][1], 0, 0, 0);
  }
  // Epilogue: GELU and W2 on the accumulators, then the sum over this tile's 32 j.
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + a * 16 + (lane >> 4) * 4 + i;
      if (j < m) {
        const float bias = b1 ? b1[j] : 0.f;
        const float w2 = bf16_to_f32(W2[j]);
#pragma unroll
        for (int c = 0; c < 2; ++c) s[c] += w2 * gelu(acc[a][c][i] + bias);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    s[c] += __shfl_xor(s[c], 16);
    s[c] += __shfl_xor(s[c], 32);
    const int b = bb0 + c * 16 + r;
    if (lane < 16 && b < B) part[static_cast<int64_t>(b) * P + blockIdx.x] = s[c];
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
  return mfma ? (m + kTileJ - 1) / kTileJ : m;
}

hipError_t launch_router_gemv(const void* hidden, int dtype, int32_t B, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, float* part,
                              hipStream_t stream) {
  const dim3 grid((m + kWaves - 1) / kWaves, (B + kGemvBatch - 1) / kGemvBatch);
  if (dtype == WF_BF16)
    hipLaunchKernelGGL(router_gemv_kernel<WF_BF16>, grid, dim3(kThreads), 0, stream, hidden, B, d,
                       W1, b1, m, W2, part);
  else
    hipLaunchKernelGGL(router_gemv_kernel<WF_F32>, grid, dim3(kThreads), 0, stream, hidden, B, d,
                       W1, b1, m, W2, part);
  return hipGetLastError();
}

hipError_t launch_router_mfma(const void* hidden, int32_t B, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, float* part,
                              hipStream_t stream) {
  const int P = (m + kTileJ - 1) / kTileJ;
  const dim3 grid(P, (B + kTileB - 1) / kTileB);
  hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(64), 0, stream,
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
