// Workgroup numbering of a launch that runs the argmax sweep's chunks and the
// router's first-layer tiles side by side.
//
// Workgroups are handed to the 8 XCDs round robin (workgroup i to XCD i % 8, as
// its local workgroup i / 8).  Of a grid of n = S + 8 r workgroups, each XCD
// runs r router tiles, at local positions s - 1, 2 s - 1, ..., r s - 1, and the
// sweep's chunks in the rest of its positions.  The chunks keep the sweep's own
// order: XCD x sweeps one contiguous range of them, in increasing order.
// Spacing the router tiles out lets each share the CUs with chunks that stream
// from HBM, instead of delaying the sweep by a launch of its own.
//
// Requires r >= 1, s >= 1 and r * s <= n / 8, so every XCD holds all its router
// positions.  The map is a bijection from [0, n) onto the S chunks and the 8 r
// tiles (checked exhaustively on the host by the sanitizer driver).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace wf {

constexpr int kXcdCount = 8;  // accelerator complex dies of an MI355X

// Spacing of the router tiles for a grid of n workgroups with r tiles per XCD,
// placed within the first `percent` of every XCD's positions (at least 1).
__host__ __device__ inline int64_t interleave_spacing(int64_t n, int64_t r, int percent) {
  const int64_t span = n / kXcdCount * percent / 100;
  const int64_t s = r > 0 ? span / r : 1;
  return s > 0 ? s : 1;
}

// Workgroup i of the grid: returns c >= 0 for sweep chunk c, or -(t + 1) for
// router tile t (t in [0, 8 r)).
__host__ __device__ inline int64_t interleave_map(int64_t i, int64_t n, int64_t r, int64_t s) {
  const int64_t x = i % kXcdCount, k = i / kXcdCount;
  const int64_t nr = (k + 1) / s;  // router positions at or before local position k
  if ((k + 1) % s == 0 && nr <= r) return -(x * r + (nr - 1)) - 1;
  const int64_t q = k - (nr < r ? nr : r);
  const int64_t per = n / kXcdCount, extra = n % kXcdCount;
  return x * (per - r) + (x < extra ? x : extra) + q;
}

}  // namespace wf
