// Element access shared by the streaming kernels over logits rows: 16-byte
// vectors of bfloat16 (8 per vector) or float32 (4 per vector), widened
// exactly to float32.
#pragma once

#include <hip/hip_runtime.h>

#include "whiflash.h"

namespace wf {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
struct Elem;

template <>
struct Elem<WF_BF16> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
  // bfloat16 is the high half of a binary32 word: widening is exact.
  __device__ static inline float lo(unsigned w) { return __uint_as_float(w << 16); }
  __device__ static inline float hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static inline float vmax(u32x4 v) {
    float a = fmaxf(fmaxf(lo(v.x), hi(v.x)), lo(v.y));
    float b = fmaxf(fmaxf(hi(v.y), lo(v.z)), hi(v.z));
    float c = fmaxf(fmaxf(lo(v.w), hi(v.w)), a);
    return fmaxf(b, c);
  }
  // First element of the vector equal to `m` (0 if none, e.g. NaN input).
  __device__ static inline int first_equal(u32x4 v, float m) {
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
    int j = 0;
#pragma unroll
    for (int k = 7; k >= 0; --k) {
      const float x = (k & 1) ? hi(w[k >> 1]) : lo(w[k >> 1]);
      if (x == m) j = k;
    }
    return j;
  }
  // Element k (0..7) of the vector, in index order.
  __device__ static inline float at(u32x4 v, int k) {
    const unsigned w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
    return (k & 1) ? hi(w) : lo(w);
  }
  __device__ static inline float scalar(const unsigned char* row, int e) {
    const unsigned short b = reinterpret_cast<const unsigned short*>(row)[e];
    return __uint_as_float(static_cast<unsigned>(b) << 16);
  }
};

template <>
struct Elem<WF_F32> {
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
  __device__ static inline float vmax(u32x4 v) {
    return fmaxf(fmaxf(__uint_as_float(v.x), __uint_as_float(v.y)),
                 fmaxf(__uint_as_float(v.z), __uint_as_float(v.w)));
  }
  __device__ static inline int first_equal(u32x4 v, float m) {
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
    int j = 0;
#pragma unroll
    for (int k = 3; k >= 0; --k)
      if (__uint_as_float(w[k]) == m) j = k;
    return j;
  }
  __device__ static inline float at(u32x4 v, int k) {
    return __uint_as_float(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
  }
  __device__ static inline float scalar(const unsigned char* row, int e) {
    return reinterpret_cast<const float*>(row)[e];
  }
};

// Streaming 16-byte load that does not allocate in the caches.
__device__ inline u32x4 load16(const u32x4* p) { return __builtin_nontemporal_load(p); }

}  // namespace wf
