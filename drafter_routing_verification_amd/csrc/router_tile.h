// A lean router stage-1 tile for launches shared with the argmax sweep (WhiFlash
// paper, section 3.3.2 and Appendix A: z = W1 h before the GELU): the same
// 32 (hidden units) x 64 (sequences) tile and the same sequence of
// v_mfma_f32_16x16x32_bf16 steps over one slice of the hidden size as
// router_mfma_kernel, so its partial sums are bitwise the same.  It differs in
// how operands reach the matrix cores: 64 columns at a time through 15 KiB of
// LDS, with the next 64 columns' loads in flight while the current ones are
// multiplied, so it needs few registers and little LDS and does not lower the
// occupancy of the sweep's workgroups in the same launch.
#pragma once

#include "common.h"
#include "elem.h"

namespace wf {

constexpr int kTileJ = 32;                                 // hidden units per tile
constexpr int kTileB = 64;                                 // sequences per tile
constexpr int kLeanChunk = 64;                             // columns staged per step
constexpr int kLeanRows = kTileJ + kTileB;                 // W1 rows, then hidden rows
constexpr int kLeanStride = kLeanChunk + 16;  // padded LDS row (elements): no bank conflicts
constexpr int kLeanPieces = kLeanRows * (kLeanChunk / 8) / kThreads;  // 16-byte pieces per thread
static_assert(kLeanPieces * kThreads == kLeanRows * (kLeanChunk / 8), "pieces must tile the chunk");

struct LeanStage {
  unsigned short s[kLeanRows * kLeanStride];
};

typedef __bf16 lean_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lean_f32x4 __attribute__((ext_vector_type(4)));

// Tile t = (jt, bt, slice) with jt fastest: hidden units [32 jt, 32 jt + 32),
// sequences [64 bt, 64 bt + 64), hidden columns [slice * kslice, ...), kslice a
// multiple of 64 and d a multiple of 8 (16-byte rows).  Writes zp[slice][b][j]
// for the tile's valid (b, j).  Tiles past the last slice do nothing.  Operand
// layout of the MFMA as in router_mfma_kernel: lane l supplies row l % 16 of the
// A and B fragments, 8 consecutive k from 8 * (l / 16).
__device__ inline void router_lean_tile(int t, int tiles_j, int tiles_b, int KS,
                                        const unsigned short* __restrict__ hidden, int B, int d,
                                        const unsigned short* __restrict__ W1, int m, int kslice,
                                        float* __restrict__ zp, LeanStage& st) {
  const int jt = t % tiles_j;
  const int bt = (t / tiles_j) % tiles_b;
  const int slice = t / (tiles_j * tiles_b);
  if (slice >= KS) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j0 = jt * kTileJ, bb0 = bt * kTileB;
  const int k0 = slice * kslice, k1 = min(d, k0 + kslice);
  const int r = lane & 15, g = lane >> 4;
  const int a = w & 1, bq = (w >> 1) * 2;
  // Piece i of this thread: row p >> 3 of the staging area, columns (p & 7) * 8 .. + 7.
  // Rows past m or B read row 0 of W1 (always valid) and are zeroed by a select,
  // so every load is unconditional.
  const unsigned short* src[kLeanPieces];
  bool live[kLeanPieces];
  int srow[kLeanPieces], scol[kLeanPieces];
#pragma unroll
  for (int i = 0; i < kLeanPieces; ++i) {
    const int p = i * kThreads + tid;
    const int row = p >> 3;
    srow[i] = row;
    scol[i] = (p & 7) * 8;
    if (row < kTileJ) {
      live[i] = j0 + row < m;
      src[i] = live[i] ? W1 + static_cast<int64_t>(j0 + row) * d : W1;
    } else {
      live[i] = bb0 + row - kTileJ < B;
      src[i] = live[i] ? hidden + static_cast<int64_t>(bb0 + row - kTileJ) * d : W1;
    }
  }
  const int nchunks = (k1 - k0 + kLeanChunk - 1) / kLeanChunk;
  auto load_chunk = [&](int c, u32x4 (&buf)[kLeanPieces]) {
#pragma unroll
    for (int i = 0; i < kLeanPieces; ++i) {
      const int k = k0 + c * kLeanChunk + scol[i];
      const bool in = live[i] && k < k1;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src[i] + (in ? k : 0));
      const u32x4 z = {0u, 0u, 0u, 0u};
      buf[i] = in ? v : z;
    }
  };
  lean_f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  u32x4 cur[kLeanPieces], nxt[kLeanPieces];
  load_chunk(0, cur);
  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) load_chunk(c + 1, nxt);
    __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
    for (int i = 0; i < kLeanPieces; ++i)
      *reinterpret_cast<u32x4*>(&st.s[srow[i] * kLeanStride + scol[i]]) = cur[i];
    __syncthreads();
#pragma unroll
    for (int step = 0; step < kLeanChunk / 32; ++step) {
      const int col = step * 32 + g * 8;
      const lean_bf16x8 fa = __builtin_bit_cast(
          lean_bf16x8, *reinterpret_cast<const u32x4*>(&st.s[(a * 16 + r) * kLeanStride + col]));
      const lean_bf16x8 f0 = __builtin_bit_cast(
          lean_bf16x8,
          *reinterpret_cast<const u32x4*>(&st.s[(kTileJ + bq * 16 + r) * kLeanStride + col]));
      const lean_bf16x8 f1 = __builtin_bit_cast(
          lean_bf16x8,
          *reinterpret_cast<const u32x4*>(&st.s[(kTileJ + (bq + 1) * 16 + r) * kLeanStride + col]));
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f1, acc1, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kLeanPieces; ++i) cur[i] = nxt[i];
  }
  // Lane holds z partials for j = j0 + 16 a + 4 g + i (i < 4), one sequence per accumulator.
  const int jb = j0 + a * 16 + g * 4;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int b = bb0 + (bq + q) * 16 + r;
    if (b >= B) continue;
    const lean_f32x4 v = q == 0 ? acc0 : acc1;
    float* dst = zp + (static_cast<int64_t>(slice) * B + b) * m + jb;
    if ((m & 3) == 0 && jb + 3 < m) {  // 16-byte aligned: one store
      *reinterpret_cast<lean_f32x4*>(dst) = v;
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (jb + i < m) dst[i] = v[i];
  }
}

}  // namespace wf
