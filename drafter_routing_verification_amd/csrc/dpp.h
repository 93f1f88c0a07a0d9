// Cross-lane reductions with DPP lane moves (registers only, no LDS round
// trip), for the small reductions at the end of latency-bound kernels.
//
// Lane patterns used (a wave64 is four rows of 16 lanes):
//   quad_perm [1,0,3,2] / [2,3,0,1]: swap lanes 1 / 2 apart within each quad;
//   row_half_mirror / row_mirror: lane i takes lane 7 - i / 15 - i of its
//     8-lane half row / 16-lane row;
//   row_bcast:15 (rows 1 and 3) / row_bcast:31 (rows 2 and 3): lane 15 of the
//     row before / lane 31, into the lanes of the rows named.
// Lanes of rows outside a step's row mask keep their own value, so in the two
// broadcast steps they combine with themselves: harmless for max, and for sums
// and merges only in lanes that do not feed lane 63, which holds the result.
#pragma once

#include <hip/hip_runtime.h>

namespace wf {

constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf>
__device__ inline int dpp_mov(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ inline float dpp_mov(float x) {
  return __int_as_float(dpp_mov<CTRL, ROW_MASK>(__float_as_int(x)));
}

// Sum over the 64 lanes of a wave, left in lane 63 (other lanes: partial sums).
__device__ inline float wave_sum_to_lane63(float x) {
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  x += dpp_mov<kDppMirror>(x);
  x += dpp_mov<kDppBcast15, 0xa>(x);
  x += dpp_mov<kDppBcast31, 0xc>(x);
  return x;
}

// Maximum over the 64 lanes of a wave, left in lane 63.
__device__ inline int wave_max_to_lane63(int x) {
  x = max(x, dpp_mov<kDppQuadXor1>(x));
  x = max(x, dpp_mov<kDppQuadXor2>(x));
  x = max(x, dpp_mov<kDppHalfMirror>(x));
  x = max(x, dpp_mov<kDppMirror>(x));
  x = max(x, dpp_mov<kDppBcast15, 0xa>(x));
  x = max(x, dpp_mov<kDppBcast31, 0xc>(x));
  return x;
}

// XOR over the 64 lanes of a wave, left in lane 63.
__device__ inline unsigned wave_xor_to_lane63(unsigned x) {
  x ^= static_cast<unsigned>(dpp_mov<kDppQuadXor1>(static_cast<int>(x)));
  x ^= static_cast<unsigned>(dpp_mov<kDppQuadXor2>(static_cast<int>(x)));
  x ^= static_cast<unsigned>(dpp_mov<kDppHalfMirror>(static_cast<int>(x)));
  x ^= static_cast<unsigned>(dpp_mov<kDppMirror>(static_cast<int>(x)));
  x ^= static_cast<unsigned>(dpp_mov<kDppBcast15, 0xa>(static_cast<int>(x)));
  x ^= static_cast<unsigned>(dpp_mov<kDppBcast31, 0xc>(static_cast<int>(x)));
  return x;
}

// Combine (bv, bi) with the pair a DPP move brings: larger value wins, ties to
// the lower index.  Bitwise operators and selects: no short-circuit branches.
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline void dpp_better(float& bv, int& bi) {
  const float v = dpp_mov<CTRL, ROW_MASK>(bv);
  const int i = dpp_mov<CTRL, ROW_MASK>(bi);
  const bool t = (v > bv) | ((v == bv) & (i < bi));
  bv = t ? v : bv;
  bi = t ? i : bi;
}

// (max, lowest index) over the 64 lanes of a wave, left in lane 63.  The
// pairs must be totally ordered (no NaN values) for the result not to depend
// on the order of combination.
__device__ inline void wave_argmax_to_lane63(float& bv, int& bi) {
  dpp_better<kDppQuadXor1>(bv, bi);
  dpp_better<kDppQuadXor2>(bv, bi);
  dpp_better<kDppHalfMirror>(bv, bi);
  dpp_better<kDppMirror>(bv, bi);
  dpp_better<kDppBcast15, 0xa>(bv, bi);
  dpp_better<kDppBcast31, 0xc>(bv, bi);
}

}  // namespace wf
