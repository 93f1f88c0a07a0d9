// One routed speculation round (WhiFlash paper, sections 3.2 and 3.3): the
// neural router, then greedy verification of each sequence with the drafter
// the router chose.  Same results as whiflash_route followed by
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
