// Lazy catch-up bookkeeping (WhiFlash paper, section 3.4 "Lazy Catch-up"):
// per sequence, tokens accepted this round join the backlog of the drafter
// that was not used; a switch hands the incoming drafter its backlog as the
// length of its one batched catch-up prefill and clears it.  One thread per
// sequence; the backlog array is updated in place.
#include "common.h"

namespace wf {
namespace {

__global__ __launch_bounds__(kThreads) void catchup_kernel(
    int B, const int32_t* __restrict__ cur, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ nxt, int32_t* __restrict__ backlog, int32_t* __restrict__ switch_flag,
    int32_t* __restrict__ catchup_len) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= B) return;
  const int c = cur[b], n = nxt[b], a = accept_len[b];
  int sw = 0, cu = 0;
  if ((c == 0 || c == 1) && (n == 0 || n == 1)) {
    int32_t* bl = backlog + 2 * static_cast<int64_t>(b);
    if (a > 0) bl[1 - c] += a;
    if (n != c) {
      sw = 1;
      cu = bl[n];
      bl[n] = 0;
    }
  }
  if (switch_flag) switch_flag[b] = sw;
  if (catchup_len) catchup_len[b] = cu;
}

}  // namespace

hipError_t launch_catchup(int32_t B, const int32_t* cur, const int32_t* accept_len,
                          const int32_t* nxt, int32_t* backlog, int32_t* switch_flag,
                          int32_t* catchup_len, hipStream_t stream) {
  hipLaunchKernelGGL(catchup_kernel, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                     B, cur, accept_len, nxt, backlog, switch_flag, catchup_len);
  return hipGetLastError();
}

}  // namespace wf
