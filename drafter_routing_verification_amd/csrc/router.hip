// WhiFlash-Neural router (WhiFlash paper, section 3.3.2 and Appendix A):
//   dal[b] = W2 . GELU(W1 h_b + b1) + b2,  choice[b] = dal[b] > tau.
// Stage 1 writes pre-activation partial sums zp[s][b][j] of z = W1 h_b over KS
// slices s of the hidden size:
//   - router_gemv_kernel (small batches or float32, KS = 1): one wave64 per
//     hidden unit j streams row j of W1 once with coalesced 16-byte loads and
//     dots it with up to 8 hidden states, reduced across the wave by DPP moves.
//   - router_mfma_kernel (bf16 batches of 9 or more): a workgroup owns a
//     32 (j) x 64 (b) tile and one slice of the hidden size.  Its operands
//     arrive as row-contiguous 16-byte loads, a few chunks ahead, are staged
//     chunk by chunk through two LDS buffers, and are multiplied with
//     v_mfma_f32_16x16x32_bf16 (float32 accumulate).  Splitting the hidden
//     size across workgroups keeps every CU busy: at 256 sequences of
//     2560 -> 1024, two slices give 256 workgroups of 96 rows x 1280 columns
//     (240 KiB of operands each, not 480 KiB).
//   - router_mfma2_kernel: the same tile and slice worked by two groups of four
//     waves on alternate chunks, for routers too large to share the sweep's
//     launch in a fused round.
// Stage 2, router_finish_kernel, one workgroup per sequence: sums the KS
// partials, adds b1, applies GELU and W2, sums over j and adds b2, all in
// float32 and in a fixed order (bitwise reproducible), then thresholds.
#include <math.h>

#include "common.h"
#include "gemv_body.h"
#include "router_math.h"

namespace wf {
namespace {

constexpr int kMfmaTileJ = 32;      // hidden units per MFMA workgroup tile
constexpr int kMfmaTileB = 64;      // sequences per MFMA workgroup tile
constexpr int kChunk = 128;         // hidden-size columns staged through LDS at a time
constexpr int kStageRows = kMfmaTileJ + kMfmaTileB;
// Rows padded by 16 elements (288 bytes apart): no LDS bank conflicts in the
// staging writes or the fragment reads.  Padded by 8, 24 or 32 elements, the
// SQ_LDS_BANK_CONFLICT counter read a third of the LDS's active cycles (256
// sequences of 2560 -> 1024: 368,640 of 1,105,920; padded by 16: 0 of 737,280).
constexpr int kStageStride = kChunk + 16;
constexpr int kPiecesPerThread = kStageRows * (kChunk / 8) / kThreads;  // 16-byte pieces
// Chunks whose loads are in flight at once: the next kRing - 1 chunks load while
// one is staged and multiplied.  Kernel trace of router stage 1 on 256 sequences
// of 2560 -> 1024 (median, one box): the earlier form (batches of 5 chunks loaded
// together through flat pointers, then staged one by one, two barriers per
// chunk) 10.68 us; this form with two LDS buffers and one barrier per chunk, 3 /
// 4 / 5 chunks in flight: 8.68 / 8.88 / 9.08 us; one LDS buffer, 3 / 4 in
// flight: 9.24 / 9.36 us.  Another box: 10.28 -> 9.44 us (m = 1024), 7.36 ->
// 6.56 us (m = 320).  The bench steps moved less than their spread.
#ifndef WF_ROUTER_RING
#define WF_ROUTER_RING 3
#endif
constexpr int kRing = WF_ROUTER_RING;
#ifndef WF_ROUTER_WGS
#define WF_ROUTER_WGS 256
#endif
// MFMA grid size the slicing of the hidden size aims for.  On 256 sequences of
// 2560 -> 1024 (bench step, same process, two interleaved trials, the kernel
// before its ring of chunks): 256 workgroups (2 slices) route 15.8 us; 512 (4
// slices, two per CU, each with one load batch) 15.6 us and the same step
// time; 1024 (7 slices) 19.0 us.  With the ring, kernel trace: 256 workgroups
// 9.12-9.36 us, 512 9.28-9.72 us, 1024 12.08 us.
constexpr int64_t kRouterWorkgroups = WF_ROUTER_WGS;
// Smallest bf16 batch routed on MFMA tiles; smaller batches (and float32) take the GEMV.
// Same box, whole whiflash_round_chain step over 151,936-wide rows, hidden 2560, m = 1024
// (m = 320), median of three trials, GEMV -> MFMA, each router in a launch of its own:
// 9 sequences 21.4 -> 21.3 us (20.9 -> 21.3); 10: 22.0 -> 21.1 (21.6 -> 21.2); 12: 24.0
// -> 21.2 (22.9 -> 21.4); 15: 26.7 -> 23.0 (25.4 -> 22.9); 16: 27.4 -> 23.6 (25.9 ->
// 23.3); 32: 41.7 -> 35.7; 256: 248.9 -> 213.1 (216.5 -> 200.3).  With small MFMA
// routers sharing the sweep's launch (round.hip), two trials: 9 sequences 21.2-21.4 ->
// 17.9 us (20.8-21.1 -> 17.9); up to 8 sequences, where the GEMV tiles share the sweep's
// launch too, the GEMV stays 0.1-0.3 us ahead (1, 2, 4 and 8 sequences measured).
#ifndef WF_ROUTER_MFMA_MIN_BATCH
#define WF_ROUTER_MFMA_MIN_BATCH 9
#endif
constexpr int32_t kMfmaMinBatch = WF_ROUTER_MFMA_MIN_BATCH;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One wave per hidden unit j and NB sequences (gemv_tile in gemv_body.h).
template <int DT, int NB, bool VEC>
__global__ __launch_bounds__(kThreads) void router_gemv_kernel(
    const void* __restrict__ hidden, HiddenSel sel, int B, int d, const void* __restrict__ W1, int m,
    float* __restrict__ zp, ZeroFill zero) {
  zero_fill_first_block(zero);
  gemv_tile<DT, NB, VEC>(blockIdx.x, blockIdx.y, hidden, sel, B, d, W1, m, zp);
}

// One workgroup = 4 waves per 32 (j) x 64 (b) tile of z^T and one slice
// [k0, k1) of the hidden size.  Rows 0..31 of a staging buffer hold W1 rows
// j0.., rows 32..95 hold hidden rows bb0..; each row chunk is kChunk wide.
// Wave w computes the 16 x 16 accumulators (j-subtile w & 1) x (b-subtiles
// 2 (w >> 1) and 2 (w >> 1) + 1).
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of
// the A tile and column (l % 16) of the B tile, 8 consecutive k values starting
// at 8 * (l / 16); the accumulator of lane l holds rows 4 * (l / 16) + i,
// i = 0..3, of column l % 16.
//
// Operands stream through a ring of kRing chunks held in registers: chunk c is
// staged into LDS buffer c & 1 while chunks c + 1 .. c + kRing - 1 are still
// loading, and its slot is refilled with chunk c + kRing right after the
// barrier.  Two buffers need one barrier per chunk: a wave writes buffer c & 1
// only after the barrier of chunk c - 1, which every wave reaches after its
// multiplies of chunk c - 2.  The loads go through global (not flat) pointers,
// so waiting on LDS traffic never waits on them.
// NCH > 0: no slice has more than NCH chunks, and the chunk loop is unrolled
// whole, so each wait names exactly the loads it needs (in a loop the compiler
// waits for every load at the top of each pass).  NCH == 0: the count is read
// at run time.
template <int NCH>
__global__ __launch_bounds__(kThreads) void router_mfma_kernel(
    const unsigned short* __restrict__ hidden, HiddenSel sel, int B, int d,
    const unsigned short* __restrict__ W1, int m, int kslice, float* __restrict__ zp,
    ZeroFill zero) {
  typedef const __attribute__((address_space(1))) u32x4 global_u32x4;
  zero_fill_first_block(zero);
  __shared__ __attribute__((aligned(16))) unsigned short stage[2][kStageRows * kStageStride];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j0 = blockIdx.x * kMfmaTileJ, bb0 = blockIdx.y * kMfmaTileB, slice = blockIdx.z;
  const int k0 = slice * kslice, k1 = min(d, k0 + kslice);
  const int r = lane & 15, g = lane >> 4;
  const int a = w & 1, bq = (w >> 1) * 2;
  // Rows this thread stages: row = i * 16 + (tid >> 4), piece column tid & 15.
  const int prow = tid >> 4, pcol = (tid & 15) * 8;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // Source row of each piece this thread stages.  Rows past m or B (or without
  // a hidden row) read row 0 of W1, always valid, and are staged as zeros.
  const unsigned short* src[kPiecesPerThread];
  bool live[kPiecesPerThread];
#pragma unroll
  for (int i = 0; i < kPiecesPerThread; ++i) {
    const int row = i * 16 + prow;
    if (row < kMfmaTileJ) {
      live[i] = j0 + row < m;
      src[i] = live[i] ? W1 + static_cast<int64_t>(j0 + row) * d : W1;
    } else {
      const int b = bb0 + row - kMfmaTileJ;
      const int64_t h = b < B ? hidden_row(sel, b) : -1;
      live[i] = h >= 0;
      src[i] = live[i] ? hidden + h * d : W1;
    }
  }
  const int nreal = (k1 - k0 + kChunk - 1) / kChunk;  // this slice's chunks
  const int nchunks = NCH > 0 ? NCH : nreal;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto in_range = [&](int c, int i) { return live[i] && c < nreal && k0 + c * kChunk + pcol < k1; };
  // Loads are unconditional (a clamped address where the piece is out of
  // range); the range is applied when the chunk is staged, so nothing waits
  // on a load before its data is staged.
  auto load = [&](int c, u32x4 (&slot)[kPiecesPerThread]) {
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) {
      const int k = in_range(c, i) ? k0 + c * kChunk + pcol : 0;
      slot[i] = *reinterpret_cast<global_u32x4*>(reinterpret_cast<uintptr_t>(src[i] + k));
    }
  };
  auto chunk = [&](int c, u32x4 (&slot)[kPiecesPerThread]) {
    unsigned short* st = stage[c & 1];
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i)
      *reinterpret_cast<u32x4*>(&st[(i * 16 + prow) * kStageStride + pcol]) =
          in_range(c, i) ? slot[i] : zero4;
    __syncthreads();
    if (c + kRing < nchunks) load(c + kRing, slot);
    if (c >= nreal) return;  // a shorter last slice: nothing to multiply
#pragma unroll
    for (int stp = 0; stp < kChunk / 32; ++stp) {
      const int col = stp * 32 + g * 8;
      const bf16x8 fa = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(&st[(a * 16 + r) * kStageStride + col]));
      const bf16x8 f0 = __builtin_bit_cast(
          bf16x8,
          *reinterpret_cast<const u32x4*>(&st[(kMfmaTileJ + bq * 16 + r) * kStageStride + col]));
      const bf16x8 f1 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(
                      &st[(kMfmaTileJ + (bq + 1) * 16 + r) * kStageStride + col]));
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f1, acc1, 0, 0, 0);
    }
  };
  u32x4 ring[kRing][kPiecesPerThread];
#pragma unroll
  for (int q = 0; q < kRing; ++q) load(q, ring[q]);
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += kRing)
#pragma unroll
      for (int q = 0; q < kRing; ++q)
        if (c0 + q < NCH) chunk(c0 + q, ring[q]);
  } else {
    for (int c0 = 0; c0 < nchunks; c0 += kRing)
#pragma unroll
      for (int q = 0; q < kRing; ++q)
        if (c0 + q < nchunks) chunk(c0 + q, ring[q]);
  }
  // z partials: lane holds j = j0 + 16a + 4g + i for one b per accumulator, so one
  // 16-byte store per accumulator when m is a multiple of 4 (the rows of zp are then
  // 16-byte aligned).  Kernel trace, 256 sequences of 2560 -> 1024: 8.64-8.72 us
  // with four 4-byte stores, 8.00-8.08 us with one 16-byte store (7.36 us with no
  // store at all).
  const int jb = j0 + a * 16 + g * 4;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int b = bb0 + (bq + q) * 16 + r;
    if (b >= B) continue;
    const f32x4 v = q == 0 ? acc0 : acc1;
    float* dst = zp + (static_cast<int64_t>(slice) * B + b) * m + jb;
    if ((m & 3) == 0 && jb + 3 < m) {
      *reinterpret_cast<f32x4*>(dst) = v;
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (jb + i < m) dst[i] = v[i];
  }
}

// The same tile and slice with two groups of four waves (512 threads): group g
// stages and multiplies the slice's chunks g, g + 2, g + 4, ... into a partial
// tile of its own, through two LDS buffers of its own, so each barrier lets two
// chunks proceed; the two partial tiles are added at the end (group 0's plus
// group 1's).  The chunk time of the one-group kernel is the chain wait -> LDS
// writes -> barrier -> LDS reads -> MFMAs that its waves walk in step; two
// groups overlap two such chains.  Kernel trace, 256 sequences of 2560 -> 1024,
// operands evicted, two runs each: 8.58-8.60 -> 7.96-8.00 us.  Its sums are
// ordered differently from router_mfma_kernel's, which the shared launch's lean
// tile reproduces, so it serves only routers too large for that launch.
template <int NCH>
__global__ __launch_bounds__(2 * kThreads) void router_mfma2_kernel(
    const unsigned short* __restrict__ hidden, HiddenSel sel, int B, int d,
    const unsigned short* __restrict__ W1, int m, int kslice, float* __restrict__ zp,
    ZeroFill zero) {
  static_assert(NCH > 0, "the chunk loop is unrolled whole");
  typedef const __attribute__((address_space(1))) u32x4 global_u32x4;
  zero_fill_first_block(zero);
  __shared__ __attribute__((aligned(16))) unsigned short stage[4][kStageRows * kStageStride];
  const int tid = threadIdx.x & (kThreads - 1), grp = threadIdx.x / kThreads;
  const int lane = tid & 63, w = tid >> 6;
  const int j0 = blockIdx.x * kMfmaTileJ, bb0 = blockIdx.y * kMfmaTileB, slice = blockIdx.z;
  const int k0 = slice * kslice, k1 = min(d, k0 + kslice);
  const int r = lane & 15, g = lane >> 4;
  const int a = w & 1, bq = (w >> 1) * 2;
  const int prow = tid >> 4, pcol = (tid & 15) * 8;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const unsigned short* src[kPiecesPerThread];
  bool live[kPiecesPerThread];
#pragma unroll
  for (int i = 0; i < kPiecesPerThread; ++i) {
    const int row = i * 16 + prow;
    if (row < kMfmaTileJ) {
      live[i] = j0 + row < m;
      src[i] = live[i] ? W1 + static_cast<int64_t>(j0 + row) * d : W1;
    } else {
      const int b = bb0 + row - kMfmaTileJ;
      const int64_t h = b < B ? hidden_row(sel, b) : -1;
      live[i] = h >= 0;
      src[i] = live[i] ? hidden + h * d : W1;
    }
  }
  const int nreal = (k1 - k0 + kChunk - 1) / kChunk;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto in_range = [&](int c, int i) { return live[i] && c < nreal && k0 + c * kChunk + pcol < k1; };
  auto load = [&](int c, u32x4 (&slot)[kPiecesPerThread]) {
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) {
      const int k = in_range(c, i) ? k0 + c * kChunk + pcol : 0;
      slot[i] = *reinterpret_cast<global_u32x4*>(reinterpret_cast<uintptr_t>(src[i] + k));
    }
  };
  constexpr int kSteps = (NCH + 1) / 2;  // steps of two chunks, one per group
  constexpr int kGroupRing = 2;          // chunks of a group in flight
  u32x4 ring[kGroupRing][kPiecesPerThread];
#pragma unroll
  for (int q = 0; q < kGroupRing; ++q) load(2 * q + grp, ring[q]);
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int q = step % kGroupRing;
    const int c = 2 * step + grp;
    // A group rewrites a buffer two steps after it last read it, and every wave
    // has passed the barrier in between.
    unsigned short* st = stage[grp * 2 + (step & 1)];
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i)
      *reinterpret_cast<u32x4*>(&st[(i * 16 + prow) * kStageStride + pcol]) =
          in_range(c, i) ? ring[q][i] : zero4;
    __syncthreads();
    if (c + 2 * kGroupRing < 2 * kSteps) load(c + 2 * kGroupRing, ring[q]);
    if (c >= nreal) continue;  // an odd chunk count: group 1's last step is empty
#pragma unroll
    for (int stp = 0; stp < kChunk / 32; ++stp) {
      const int col = stp * 32 + g * 8;
      const bf16x8 fa = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(&st[(a * 16 + r) * kStageStride + col]));
      const bf16x8 f0 = __builtin_bit_cast(
          bf16x8,
          *reinterpret_cast<const u32x4*>(&st[(kMfmaTileJ + bq * 16 + r) * kStageStride + col]));
      const bf16x8 f1 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(
                      &st[(kMfmaTileJ + (bq + 1) * 16 + r) * kStageStride + col]));
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, f1, acc1, 0, 0, 0);
    }
  }
  // Group 1 hands its partial tile to group 0 through the first buffer.
  __syncthreads();
  f32x4* handoff = reinterpret_cast<f32x4*>(&stage[0][0]);
  if (grp == 1) {
    handoff[(w * 2 + 0) * 64 + lane] = acc0;
    handoff[(w * 2 + 1) * 64 + lane] = acc1;
  }
  __syncthreads();
  if (grp == 1) return;
  acc0 = acc0 + handoff[(w * 2 + 0) * 64 + lane];
  acc1 = acc1 + handoff[(w * 2 + 1) * 64 + lane];
  const int jb = j0 + a * 16 + g * 4;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int b = bb0 + (bq + q) * 16 + r;
    if (b >= B) continue;
    const f32x4 v = q == 0 ? acc0 : acc1;
    float* dst = zp + (static_cast<int64_t>(slice) * B + b) * m + jb;
    if ((m & 3) == 0 && jb + 3 < m) {
      *reinterpret_cast<f32x4*>(dst) = v;
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (jb + i < m) dst[i] = v[i];
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void router_finish_kernel(
    const float* __restrict__ zp, HiddenSel sel, int KS, int B, int m, const float* __restrict__ b1,
    const void* __restrict__ W2, const float* __restrict__ b2, float tau,
    float* __restrict__ delta_al, int32_t* __restrict__ choice) {
  __shared__ float red[kWaves];
  const int b = blockIdx.x;
  const float v = router_finish_sequence<DT>(zp, sel, KS, B, m, b, b1, W2, b2, red);
  if (threadIdx.x == 0) {
    delta_al[b] = v;
    choice[b] = v > tau ? 1 : 0;
  }
}

}  // namespace

RouterPlan router_plan(int dtype, int32_t B, int32_t d, int32_t m, const void* hidden,
                       const void* W1) {
  RouterPlan p{false, 1, d};
  const bool aligned = (reinterpret_cast<uintptr_t>(hidden) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(W1) % 16 == 0) && (d % 8 == 0);
  if (dtype != WF_BF16 || B < kMfmaMinBatch || !aligned) return p;
  p.mfma = true;
  // 64-bit arithmetic: the slice width is d rounded up to a multiple of kChunk.
  int64_t ks = router_max_slices(B, m);
  const int64_t max_by_d = (static_cast<int64_t>(d) + kChunk - 1) / kChunk;
  if (ks > max_by_d) ks = max_by_d;
  const int64_t per = (static_cast<int64_t>(d) + ks - 1) / ks;
  const int64_t kslice = (per + kChunk - 1) / kChunk * kChunk;
  p.kslice = static_cast<int32_t>(kslice);
  p.slices = static_cast<int32_t>((static_cast<int64_t>(d) + kslice - 1) / kslice);
  return p;
}

int32_t router_max_slices(int32_t B, int32_t m) {
  // Split the hidden size until the grid covers ~kRouterWorkgroups workgroups.
  const int64_t tiles = ((static_cast<int64_t>(m) + kMfmaTileJ - 1) / kMfmaTileJ) *
                        ((static_cast<int64_t>(B) + kMfmaTileB - 1) / kMfmaTileB);
  int64_t ks = tiles > 0 ? kRouterWorkgroups / tiles : 1;
  if (ks < 1) ks = 1;
  if (ks > kMaxRouterSlices) ks = kMaxRouterSlices;
  return static_cast<int32_t>(ks);
}

template <int DT, int NB, bool VEC>
static void gemv_launch(dim3 grid, hipStream_t stream, const void* hidden, const HiddenSel& sel,
                        int32_t B, int32_t d, const void* W1, int32_t m, float* zp, ZeroFill zero) {
  hipLaunchKernelGGL((router_gemv_kernel<DT, NB, VEC>), grid, dim3(kThreads), 0, stream, hidden, sel,
                     B, d, W1, m, zp, zero);
}

template <int DT, bool VEC>
static void gemv_dispatch(const void* hidden, const HiddenSel& sel, int32_t B, int32_t d,
                          const void* W1, int32_t m, float* zp, hipStream_t stream, ZeroFill zero) {
  const unsigned gx = (m + kWaves - 1) / kWaves;
  if (B == 1) gemv_launch<DT, 1, VEC>(dim3(gx, 1), stream, hidden, sel, B, d, W1, m, zp, zero);
  else if (B <= 2) gemv_launch<DT, 2, VEC>(dim3(gx, 1), stream, hidden, sel, B, d, W1, m, zp, zero);
  else if (B <= 4) gemv_launch<DT, 4, VEC>(dim3(gx, 1), stream, hidden, sel, B, d, W1, m, zp, zero);
  else gemv_launch<DT, 8, VEC>(dim3(gx, (B + 7) / 8), stream, hidden, sel, B, d, W1, m, zp, zero);
}

hipError_t launch_router_stage1(const RouterPlan& plan, const void* hidden, const HiddenSel& sel,
                                int dtype, int32_t B, int32_t d, const void* W1, int32_t m,
                                float* zp, hipStream_t stream, ZeroFill zero) {
  if (plan.mfma) {
    const dim3 grid((m + kMfmaTileJ - 1) / kMfmaTileJ, (B + kMfmaTileB - 1) / kMfmaTileB,
                    plan.slices);
    const unsigned short* h = static_cast<const unsigned short*>(hidden);
    const unsigned short* w1 = static_cast<const unsigned short*>(W1);
    // Two groups pay from 8 chunks per slice on; at 5 the final hand-off costs more
    // than the overlap saves (bench kernel trace, 128 sequences of 2560 -> 1024:
    // 5.76-5.88 -> 6.00 us; 256 of 4096 -> 512, 8 chunks: 8.04-8.28 -> 7.60-7.76 us;
    // 256 of 2560 -> 1024, 10 chunks: 8.96-9.36 -> 8.36-8.40 us).
    const bool two = !router_lean_tiles(plan, B, m) && plan.kslice / kChunk >= 8;
#define WF_MFMA(N)                                                                               \
  do {                                                                                           \
    if (two)                                                                                     \
      hipLaunchKernelGGL(router_mfma2_kernel<N>, grid, dim3(2 * kThreads), 0, stream, h, sel, B, \
                         d, w1, m, plan.kslice, zp, zero);                                      \
    else                                                                                         \
      hipLaunchKernelGGL(router_mfma_kernel<N>, grid, dim3(kThreads), 0, stream, h, sel, B, d,   \
                         w1, m, plan.kslice, zp, zero);                                         \
  } while (0)
    // The chunk counts of the usual slicings (2,560 or 4,096 wide hidden states
    // at 9 to 65,535 sequences); any other count takes the run-time loop.
    switch (plan.kslice / kChunk) {
      case 3: WF_MFMA(3); break;
      case 4: WF_MFMA(4); break;
      case 5: WF_MFMA(5); break;
      case 6: WF_MFMA(6); break;
      case 7: WF_MFMA(7); break;
      case 8: WF_MFMA(8); break;
      case 10: WF_MFMA(10); break;
      case 16: WF_MFMA(16); break;
      case 20: WF_MFMA(20); break;
      case 32: WF_MFMA(32); break;
      default:  // a run-time chunk count: the one-group kernel's loop
        hipLaunchKernelGGL(router_mfma_kernel<0>, grid, dim3(kThreads), 0, stream, h, sel, B, d,
                           w1, m, plan.kslice, zp, zero);
        break;
    }
#undef WF_MFMA
    return hipGetLastError();
  }
  const int per = dtype == WF_BF16 ? 8 : 4;
  const bool vec = (reinterpret_cast<uintptr_t>(hidden) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(W1) % 16 == 0) && (d % per == 0);
  if (dtype == WF_BF16) {
    if (vec) gemv_dispatch<WF_BF16, true>(hidden, sel, B, d, W1, m, zp, stream, zero);
    else gemv_dispatch<WF_BF16, false>(hidden, sel, B, d, W1, m, zp, stream, zero);
  } else {
    if (vec) gemv_dispatch<WF_F32, true>(hidden, sel, B, d, W1, m, zp, stream, zero);
    else gemv_dispatch<WF_F32, false>(hidden, sel, B, d, W1, m, zp, stream, zero);
  }
  return hipGetLastError();
}

hipError_t launch_router_finish(const RouterPlan& plan, const HiddenSel& sel, int dtype,
                                const float* zp, int32_t B, int32_t m, const float* b1,
                                const void* W2, const float* b2, float tau, float* delta_al,
                                int32_t* choice, hipStream_t stream) {
  if (dtype == WF_BF16)
    hipLaunchKernelGGL(router_finish_kernel<WF_BF16>, dim3(B), dim3(kThreads), 0, stream, zp, sel,
                       plan.slices, B, m, b1, W2, b2, tau, delta_al, choice);
  else
    hipLaunchKernelGGL(router_finish_kernel<WF_F32>, dim3(B), dim3(kThreads), 0, stream, zp, sel,
                       plan.slices, B, m, b1, W2, b2, tau, delta_al, choice);
  return hipGetLastError();
}

}  // namespace wf
