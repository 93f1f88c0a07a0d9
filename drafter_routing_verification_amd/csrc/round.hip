// One routed speculation round (WhiFlash paper, sections 3.2 and 3.3): the
// neural router, then greedy verification of each sequence with the drafter
// the router chose.  Also the chain-only round: the router (its choice is for
// the next round) and the DFlash verification, sharing one final kernel.  Same results as whiflash_route followed by
// whiflash_verify_routed, in three launches instead of four: router stage 1,
// the argmax sweep, then one kernel per sequence that finishes the router
// (Delta-AL and the drafter choice) and verifies the sequence with it.
// (Running the router's workgroups inside the sweep's launch was measured
// slower: latency-bound router tiles stretched the 217 us sweep to 245 us.)
#include "accept.h"
#include "common.h"
#include "router_math.h"

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
  finish_load_pass<DT>(fin, zp, KS, B, m, b, 0, b1, W2);
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
  finish_load_pass<DT>(fin, zp, KS, B, m, b, 0, b1, W2);
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

}  // namespace

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
