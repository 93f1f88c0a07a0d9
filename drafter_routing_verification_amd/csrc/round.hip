// One routed speculation round (WhiFlash paper, sections 3.2 and 3.3): the
// neural router, then greedy verification of each sequence with the drafter
// the router chose; and the chain-only round: the router (its choice is for the
// next round) and the DFlash verification.  Same results as whiflash_route
// followed by whiflash_verify_routed (or whiflash_verify_chain), in fewer
// launches: router stage 1 and the argmax sweep, then one kernel per sequence
// that finishes the router (Delta-AL and the drafter choice) and verifies the
// sequence.
//
// Router stage 1 takes one of three forms:
//   - up to 8 sequences on the GEMV path: its GEMV tiles share the sweep's
//     launch (router_sweep_kernel), two launches per round;
//   - a small MFMA router (at most WF_ROUTER_INTERLEAVE_LOADS chunk loads): its
//     lean tiles share the sweep's launch, spread through the first part of every
//     XCD's workgroups (router_mfma_sweep_kernel), two launches per round;
//   - a larger one: a launch of its own (router.hip), three launches per round.
//     Its tiles inside the sweep's launch, heavy or lean, spread or trailing,
//     measured slower: under a sweep that saturates HBM they hold their slots
//     through long chains of loads.
#include "accept.h"
#include "common.h"
#include "gemv_body.h"
#include "interleave.h"
#include "router_math.h"
#include "router_tile.h"
#include "sweep_body.h"

// Router tiles of a shared launch sit within the first WF_ROUTER_INTERLEAVE
// percent of each XCD's workgroups (0: router stage 1 always gets a launch of
// its own).  Only a router of at most WF_ROUTER_INTERLEAVE_LOADS chunk loads
// (tiles x 64-column chunks per tile) shares the sweep's launch.
//
// Same box, bench step, two interleaved trials, separate launch -> shared launch
// (first 25 / 50 / 75 / 100 percent):
//   32 chains, 2560 -> 1024 (224 tiles x 6 chunks)   35.1 -> 31.0 / 31.2 / 32.5 / 33.0 us
//   128 routed, 2560 -> 1024 (256 tiles x 10 chunks)  220.1 -> 221.9 / 223.0 / 224.4 / 226.4 us
//   256 chains, 2560 -> 1024 (256 tiles x 20 chunks)  197.5 -> 203.4 / 202.7 / 202.1 / 213.3 us
// Under a sweep that saturates HBM every chunk a tile loads is a long round
// trip, and a tile holds its slot for all of them: a large router costs the
// sweep more than its own launch does.
#ifndef WF_ROUTER_INTERLEAVE
#define WF_ROUTER_INTERLEAVE 25
#endif
#ifndef WF_ROUTER_INTERLEAVE_LOADS
#define WF_ROUTER_INTERLEAVE_LOADS 2048
#endif

namespace wf {
namespace {

template <int DT>
__global__ __launch_bounds__(kThreads) void round_finalize_kernel(
    const float* __restrict__ zp, int KS, int B, int m, const float* __restrict__ b1,
    const void* __restrict__ W2, const float* __restrict__ b2, float tau,
    float* __restrict__ delta_al, int32_t* __restrict__ choice, RoutedArgs args) {
  __shared__ AcceptLds lds;
  __shared__ float redf[kWaves];
  const int b = blockIdx.x;
  const HiddenSel direct{nullptr, nullptr, 0, 0};
  // Phase 1: every load that depends on nothing else (router partials, offsets,
  // drafts, parents, draft ids); phase 2: chunk partials and d2t entries.
  RoutedIn in;
  routed_load_phase1(in, args, b);
  FinishIn fin;
  finish_load_pass<DT>(fin, zp, KS, B, m, b, 0, b1, W2, b2, direct);
  routed_load_phase2(in, args);
  const float dal = router_finish_compute<DT>(fin, zp, direct, KS, B, m, b, b1, W2, b2, redf);
  const int c = dal > tau ? 1 : 0;
  if (threadIdx.x == 0) {
    delta_al[b] = dal;
    choice[b] = c;
  }
  routed_accept(in, args, b, c, lds);
}

// One DFlash round over a chain-only batch: finish the router for sequence b
// (Delta-AL and the drafter choice for the next round) and verify its chain.
// The chain's acceptance does not depend on the choice, so both run from one
// load phase.
template <int DT>
__global__ __launch_bounds__(kThreads) void round_chain_finalize_kernel(
    const float* __restrict__ zp, int KS, int m, const float* __restrict__ b1,
    const void* __restrict__ W2, const float* __restrict__ b2, float tau,
    float* __restrict__ delta_al, int32_t* __restrict__ choice, const Partial* __restrict__ part,
    int splits, int B, int K, const int32_t* __restrict__ draft, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ bonus, int32_t* __restrict__ row_argmax) {
  __shared__ int t_s[kMaxSeqRows];
  __shared__ float redf[kWaves];
  const int b = blockIdx.x;
  const int R = K + 1;
  const HiddenSel direct{nullptr, nullptr, 0, 0};
  const int32_t* dr = draft + static_cast<int64_t>(b) * K;
  const int draft0 = K > 0 ? chain_load(dr, K) : -1;
  FinishIn fin;
  finish_load_pass<DT>(fin, zp, KS, B, m, b, 0, b1, W2, b2, direct);
  MergeIn mi;
  merge_load(mi, part, splits, b * R, R);
  merge_finish(mi, part, splits, b * R, R, t_s, row_argmax);
  const float dal = router_finish_compute<DT>(fin, zp, direct, KS, B, m, b, b1, W2, b2, redf);
  if (threadIdx.x == 0) {
    delta_al[b] = dal;
    choice[b] = dal > tau ? 1 : 0;
  }
  // router_finish_compute ends with a barrier, so t_s is complete here.
  chain_accept(draft0, t_s, K, dr, accept_len + b, bonus + b, nullptr);
}

// First launch of a small-batch round: router_blocks workgroups run the
// router's GEMV tiles (router workgroup i: hidden units 4 i .. 4 i + 3 for every
// sequence, all B <= NB of them), the rest run the argmax sweep's chunks.  The
// router's workgroups come first, or last when router_last is set (the sweep's
// chunks are then dispatched first).
// The two halves read disjoint inputs and write disjoint outputs.  At a few
// sequences both are small and latency-bound, so one launch instead of two
// saves a launch floor; at large batches the router runs on MFMA tiles in a
// launch of its own (router tiles inside the sweep's launch measured slower).
template <int DTL, int DTH, int NB>
__global__ __launch_bounds__(kThreads) void router_sweep_kernel(
    const void* __restrict__ hidden, int B, int d, const void* __restrict__ W1, int m,
    float* __restrict__ zp, int router_blocks, int router_last,
    const unsigned char* __restrict__ logits, int64_t row_bytes, int V, int splits,
    int chunk_vecs, int nvec, Partial* __restrict__ part) {
  const int nsweep = static_cast<int>(gridDim.x) - router_blocks;
  const int i = static_cast<int>(blockIdx.x) - (router_last ? nsweep : 0);  // router workgroup
  if (i >= 0 && i < router_blocks) {
    const HiddenSel direct{nullptr, nullptr, 0, 0};
    gemv_tile<DTH, NB, true>(i, 0, hidden, direct, B, d, W1, m, zp);
  } else {
    // Few rows, few workgroups per CU: each thread issues its whole batch of loads at once.
    const int c = router_last ? static_cast<int>(blockIdx.x) : i - router_blocks;
    sweep_chunk<DTL, kThreads, true>(c, logits, row_bytes, V, splits, chunk_vecs, nvec, part);
  }
}

// First launch of a round on the MFMA router path: router stage-1 tiles (lean
// form, router_tile.h) spaced through the first part of every XCD's workgroups,
// the sweep's chunks in all other positions (interleave.h).  The two kinds read
// disjoint inputs and write disjoint outputs.
template <int DTL, bool kBatch>
__global__ __launch_bounds__(kThreads) void router_mfma_sweep_kernel(
    const unsigned short* __restrict__ hidden, int B, int d, const unsigned short* __restrict__ W1,
    int m, int kslice, int KS, int tiles_j, int tiles_b, float* __restrict__ zp,
    int64_t router_per_xcd, int64_t spacing, const unsigned char* __restrict__ logits,
    int64_t row_bytes, int V, int splits, int chunk_vecs, int nvec, Partial* __restrict__ part) {
  __shared__ LeanStage stage;
  const int64_t t = interleave_map(blockIdx.x, gridDim.x, router_per_xcd, spacing);
  if (t < 0) {
    router_lean_tile(static_cast<int>(-t - 1), tiles_j, tiles_b, KS, hidden, B, d, W1, m, kslice,
                     zp, stage);
  } else if (kBatch || sweep_edge_block()) {
    sweep_chunk<DTL, kThreads, true>(static_cast<int>(t), logits, row_bytes, V, splits,
                                     chunk_vecs, nvec, part);
  } else {
    sweep_chunk<DTL, kThreads, false>(static_cast<int>(t), logits, row_bytes, V, splits,
                                      chunk_vecs, nvec, part);
  }
}

template <int DTL, int DTH>
hipError_t launch_router_sweep_nb(unsigned grid, int nb, const void* hidden, int B, int d,
                                  const void* W1, int m, float* zp, int router_blocks,
                                  int router_last, const unsigned char* logits, int64_t row_bytes,
                                  int V,
                                  int splits, int chunk_vecs, int nvec, Partial* part,
                                  hipStream_t stream) {
#define WF_ROUTER_SWEEP(NBV)                                                                   \
  hipLaunchKernelGGL((router_sweep_kernel<DTL, DTH, NBV>), dim3(grid), dim3(kThreads), 0, stream, \
                     hidden, B, d, W1, m, zp, router_blocks, router_last, logits, row_bytes, V, \
                     splits, chunk_vecs, nvec, part)
  if (nb == 1) WF_ROUTER_SWEEP(1);
  else if (nb == 2) WF_ROUTER_SWEEP(2);
  else if (nb == 4) WF_ROUTER_SWEEP(4);
  else WF_ROUTER_SWEEP(8);
#undef WF_ROUTER_SWEEP
  return hipGetLastError();
}

}  // namespace

bool router_lean_tiles(const RouterPlan& plan, int32_t B, int32_t m) {
  if (WF_ROUTER_INTERLEAVE <= 0 || !plan.mfma || plan.kslice % kLeanChunk != 0) return false;
  const int64_t tiles = static_cast<int64_t>((m + kTileJ - 1) / kTileJ) *
                        ((B + kTileB - 1) / kTileB) * plan.slices;
  return tiles * (plan.kslice / kLeanChunk) <= WF_ROUTER_INTERLEAVE_LOADS;
}

bool round_stage1_fused(const RouterPlan& plan, int hidden_dtype, const void* hidden, int32_t B,
                        int32_t d, const void* W1) {
  const int per_h = hidden_dtype == WF_BF16 ? 8 : 4;
  const bool vec = (reinterpret_cast<uintptr_t>(hidden) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(W1) % 16 == 0) && (d % per_h == 0);
  return !plan.mfma && vec && B <= 8;
}

SweepPlan few_rows_plan(int32_t rows, int32_t V, int32_t rows_per_seq) {
  // The final kernel merges a sequence's partials with groups of G lanes per row
  // (G a power of two), 256 / G rows per pass, kMergePer partials per lane.  With
  // at most kMergePer * G chunks per row and G <= 256 / rows_per_seq, every row
  // of a sequence is merged in the first pass, from one round of loads.
  SweepPlan p = sweep_plan(rows, V);
  int G = 1;
  while (2 * G * (rows_per_seq > 0 ? rows_per_seq : 1) <= kThreads && G < 64) G <<= 1;
  const int cap = kMergePer * G;
  if (p.splits > cap) {
    int64_t chunk = (static_cast<int64_t>(V) + cap - 1) / cap;
    chunk = (chunk + 255) / 256 * 256;
    p.chunk = static_cast<int32_t>(chunk);
    p.splits = static_cast<int32_t>((V + chunk - 1) / chunk);
  }
  return p;
}

namespace {

// Router stage 1 (MFMA path) and the sweep in one launch, tiles interleaved.
template <int DTL>
hipError_t launch_router_mfma_sweep(const RouterPlan& plan, const void* hidden, int32_t B, int32_t d,
                                    const void* W1, int32_t m, float* zp, const void* logits,
                                    int64_t row_stride, int32_t rows, int32_t V, SweepPlan sp,
                                    Partial* part, int64_t r, hipStream_t stream) {
  using E = Elem<DTL>;
  const int tiles_j = (m + kTileJ - 1) / kTileJ, tiles_b = (B + kTileB - 1) / kTileB;
  const int64_t sweep_blocks = static_cast<int64_t>(rows) * sp.splits;
  const int64_t n = sweep_blocks + kXcdCount * r;
  const int64_t s = interleave_spacing(n, r, WF_ROUTER_INTERLEAVE);
  const unsigned char* base = static_cast<const unsigned char*>(logits);
  const int64_t rb = row_stride * E::kBytes;
  const int cv = sp.chunk / E::kPerVec, nv = V / E::kPerVec;
  const unsigned short* h = static_cast<const unsigned short*>(hidden);
  const unsigned short* w = static_cast<const unsigned short*>(W1);
  if (sweep_batched(sweep_blocks))
    hipLaunchKernelGGL((router_mfma_sweep_kernel<DTL, true>), dim3(static_cast<unsigned>(n)),
                       dim3(kThreads), 0, stream, h, B, d, w, m, plan.kslice, plan.slices, tiles_j,
                       tiles_b, zp, r, s, base, rb, V, sp.splits, cv, nv, part);
  else
    hipLaunchKernelGGL((router_mfma_sweep_kernel<DTL, false>), dim3(static_cast<unsigned>(n)),
                       dim3(kThreads), 0, stream, h, B, d, w, m, plan.kslice, plan.slices, tiles_j,
                       tiles_b, zp, r, s, base, rb, V, sp.splits, cv, nv, part);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_round_stage1(bool fused, const RouterPlan& plan, int hidden_dtype,
                               const void* hidden, int32_t B, int32_t d, const void* W1, int32_t m,
                               float* zp, const void* logits, int logits_dtype, int64_t row_stride,
                               int32_t rows, int32_t V, SweepPlan sp, Partial* part,
                               hipStream_t stream) {
  const int64_t router_gx = (static_cast<int64_t>(m) + kWaves - 1) / kWaves;
  const int64_t sweep_blocks = static_cast<int64_t>(rows) * sp.splits;
  if (router_lean_tiles(plan, B, m)) {
    // Router tiles padded to a whole number per XCD; the padding tiles do nothing.
    const int64_t tiles = static_cast<int64_t>((m + kTileJ - 1) / kTileJ) *
                          ((B + kTileB - 1) / kTileB) * plan.slices;
    const int64_t r = (tiles + kXcdCount - 1) / kXcdCount;
    if (sweep_blocks + kXcdCount * r <= INT32_MAX && sweep_blocks / kXcdCount >= r) {
      return logits_dtype == WF_BF16
                 ? launch_router_mfma_sweep<WF_BF16>(plan, hidden, B, d, W1, m, zp, logits,
                                                     row_stride, rows, V, sp, part, r, stream)
                 : launch_router_mfma_sweep<WF_F32>(plan, hidden, B, d, W1, m, zp, logits,
                                                    row_stride, rows, V, sp, part, r, stream);
    }
  }
  if (!fused || router_gx + sweep_blocks > INT32_MAX) {
    const HiddenSel direct{nullptr, nullptr, 0, 0};
    if (launch_router_stage1(plan, hidden, direct, hidden_dtype, B, d, W1, m, zp, stream) !=
        hipSuccess)
      return hipErrorLaunchFailure;
    return launch_sweep(logits, logits_dtype, row_stride, rows, V, sp, part, stream);
  }
  const int nb = B == 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8;
  // One sequence: its sweep chunks are dispatched ahead of the router's tiles.
  const int last = B == 1 ? 1 : 0;
  const unsigned grid = static_cast<unsigned>(router_gx + sweep_blocks);
  const unsigned char* base = static_cast<const unsigned char*>(logits);
  const int gx = static_cast<int>(router_gx);
  const bool bf16_logits = logits_dtype == WF_BF16;
  const int per = bf16_logits ? Elem<WF_BF16>::kPerVec : Elem<WF_F32>::kPerVec;
  const int64_t rb = row_stride * (bf16_logits ? Elem<WF_BF16>::kBytes : Elem<WF_F32>::kBytes);
  const int cv = sp.chunk / per, nv = V / per;
#define WF_STAGE1(DTL, DTH)                                                                      \
  launch_router_sweep_nb<DTL, DTH>(grid, nb, hidden, B, d, W1, m, zp, gx, last, base, rb, V,   \
                                   sp.splits, cv, nv, part, stream)
  if (bf16_logits)
    return hidden_dtype == WF_BF16 ? WF_STAGE1(WF_BF16, WF_BF16) : WF_STAGE1(WF_BF16, WF_F32);
  return hidden_dtype == WF_BF16 ? WF_STAGE1(WF_F32, WF_BF16) : WF_STAGE1(WF_F32, WF_F32);
#undef WF_STAGE1
}

hipError_t launch_round_finalize(int hidden_dtype, const RouterPlan& plan, const float* zp, int32_t B,
                                 int32_t m, const float* b1, const void* W2, const float* b2,
                                 float tau, float* delta_al, int32_t* choice,
                                 const RoutedArgs& args, hipStream_t stream) {
  if (hidden_dtype == WF_BF16)
    hipLaunchKernelGGL(round_finalize_kernel<WF_BF16>, dim3(B), dim3(kThreads), 0, stream, zp,
                       plan.slices, B, m, b1, W2, b2, tau, delta_al, choice, args);
  else
    hipLaunchKernelGGL(round_finalize_kernel<WF_F32>, dim3(B), dim3(kThreads), 0, stream, zp,
                       plan.slices, B, m, b1, W2, b2, tau, delta_al, choice, args);
  return hipGetLastError();
}

}  // namespace wf

namespace wf {

hipError_t launch_round_chain_finalize(int hidden_dtype, const RouterPlan& plan, const float* zp,
                                       int32_t B, int32_t m, const float* b1, const void* W2,
                                       const float* b2, float tau, float* delta_al,
                                       int32_t* choice, const Partial* part, int32_t splits,
                                       int32_t K, const int32_t* draft, int32_t* accept_len,
                                       int32_t* bonus, int32_t* row_argmax, hipStream_t stream) {
  if (hidden_dtype == WF_BF16)
    hipLaunchKernelGGL(round_chain_finalize_kernel<WF_BF16>, dim3(B), dim3(kThreads), 0, stream,
                       zp, plan.slices, m, b1, W2, b2, tau, delta_al, choice, part, splits, B, K,
                       draft, accept_len, bonus, row_argmax);
  else
    hipLaunchKernelGGL(round_chain_finalize_kernel<WF_F32>, dim3(B), dim3(kThreads), 0, stream,
                       zp, plan.slices, m, b1, W2, b2, tau, delta_al, choice, part, splits, B, K,
                       draft, accept_len, bonus, row_argmax);
  return hipGetLastError();
}

}  // namespace wf
