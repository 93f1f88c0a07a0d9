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
  // Both backlog entries are loaded with the inputs, in one round trip, and
  // updated without branches; a sequence with an out-of-range choice gets its
  // entries written back unchanged.
  int32_t* bl = backlog + 2 * static_cast<int64_t>(b);
  const int c = cur[b], n = nxt[b], a = accept_len[b];
  const int x0 = bl[0], x1 = bl[1];
  const bool ok = (c == 0 || c == 1) && (n == 0 || n == 1);
  const int add = ok && a > 0 ? a : 0;
  const int y0 = x0 + (c == 1 ? add : 0);  // tokens accepted while drafter 0 was idle
  const int y1 = x1 + (c == 0 ? add : 0);
  const bool sw = ok && n != c;
  const int cu = sw ? (n == 0 ? y0 : y1) : 0;
  bl[0] = sw && n == 0 ? 0 : y0;
  bl[1] = sw && n == 1 ? 0 : y1;
  if (switch_flag) switch_flag[b] = sw ? 1 : 0;
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
