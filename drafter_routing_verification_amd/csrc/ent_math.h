// Online entropy arithmetic of the WhiFlash-Entropy policy (WhiFlash paper,
// section 3.3.1: entropy of the softmax of the target's logits row).
//
// In base 2, with y = (x - m) log2(e) for a running maximum m, a stream keeps
// S = sum of 2^y and U = sum of y 2^y.  Moving to a larger maximum m'
// multiplies every 2^y by f = 2^d, d = (m - m') log2(e), and shifts every y by
// d, so S' = S f and U' = (U + d S) f.  Partial streams merge the same way, and
// H = ln 2 (log2 S - U / S) nats.
#pragma once

#include <math.h>

#include "dpp.h"

namespace wf {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Ent {
  float m, S, U;
};

// Folds b into a (either may be empty: S == 0).
__device__ inline void ent_merge(Ent& a, const Ent& b) {
  if (b.S == 0.f) return;
  if (a.S == 0.f) {
    a = b;
    return;
  }
  const float M = fmaxf(a.m, b.m);
  const float da = (a.m - M) * kLog2e, db = (b.m - M) * kLog2e;
  const float fa = __builtin_amdgcn_exp2f(da), fb = __builtin_amdgcn_exp2f(db);
  a.U = (a.U + da * a.S) * fa + (b.U + db * b.S) * fb;
  a.S = a.S * fa + b.S * fb;
  a.m = M;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ inline void ent_dpp_merge(Ent& a) {
  const Ent o{dpp_mov<CTRL, ROW_MASK>(a.m), dpp_mov<CTRL, ROW_MASK>(a.S),
              dpp_mov<CTRL, ROW_MASK>(a.U)};
  ent_merge(a, o);
}

// Merge of the 64 lanes' streams of a wave, left in lane 63 (a fixed order).
__device__ inline void wave_ent_to_lane63(Ent& a) {
  ent_dpp_merge<kDppQuadXor1>(a);
  ent_dpp_merge<kDppQuadXor2>(a);
  ent_dpp_merge<kDppHalfMirror>(a);
  ent_dpp_merge<kDppMirror>(a);
  ent_dpp_merge<kDppBcast15, 0xa>(a);
  ent_dpp_merge<kDppBcast31, 0xc>(a);
}

// Raises the running maximum of a to mv (mv > a.m), rescaling S and U.
__device__ inline void ent_raise(Ent& a, float mv) {
  if (a.S != 0.f) {
    const float dl = (a.m - mv) * kLog2e;
    const float f = __builtin_amdgcn_exp2f(dl);
    a.U = (a.U + dl * a.S) * f;
    a.S *= f;
  }
  a.m = mv;
}

// Adds one element x (x <= a.m) given mb = a.m * log2(e).
__device__ inline void ent_add(Ent& a, float x, float mb) {
  const float y = fmaf(x, kLog2e, -mb);
  const float e = __builtin_amdgcn_exp2f(y);
  a.S += e;
  a.U = fmaf(y, e, a.U);
}

// H in nats of a merged stream; NaN when it is empty.
__device__ inline float ent_value(const Ent& a) {
  return a.S > 0.f ? kLn2 * (__builtin_amdgcn_logf(a.S) - a.U / a.S) : NAN;
}

}  // namespace wf
