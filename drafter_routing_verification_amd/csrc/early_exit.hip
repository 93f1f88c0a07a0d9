// DFlash chain verification that stops reading a sequence's logits once its
// first mismatch is known.  Decoding continues from the last accepted token
// (WhiFlash paper, section 3.2), so the rows after the first rejected draft
// change neither the acceptance length nor the bonus token; only rows 0..n of a
// sequence are needed, n being the first mismatch.
//
// Schedule.  One workgroup per chunk of a row, launched position-major (every
// sequence's row 0, then every sequence's row 1, ...), so a sequence's early
// rows are swept before its later rows are dispatched.  Each sequence keeps
// e = INT_MAX - (lowest known mismatch position) in the workspace, 0 when none
// is known.  A workgroup first reads e and skips its chunk when a mismatch at an
// earlier position is known.
//
// Detection without a row merge.  The draft token d at position i is the
// greedy token iff no element beats (x[d], d) under the argmax order (larger,
// or equal at a lower index).  So any chunk whose own maximum beats (x[d], d)
// proves a mismatch by itself, and the chunk holding the row maximum always
// does when there is one.  That chunk raises e with an agent-scope atomic max.
//
// Why stale reads are harmless.  e only ever names positions of real mismatches,
// all >= n, so rows 0..n are never skipped and their partials are exact.  A
// late or stale read of e only means a chunk that could have been skipped is
// read.  No fence is needed.  The acceptance kernel scans positions in order,
// so n and t[n] come out exact; rows after n are reported as -1.
#include "accept.h"
#include "common.h"
#include "sweep_body.h"

#ifndef WF_EARLY_EXIT_THREADS
#define WF_EARLY_EXIT_THREADS 512
#endif
#ifndef WF_EARLY_EXIT_CHUNK
#define WF_EARLY_EXIT_CHUNK (WF_EARLY_EXIT_THREADS * 64)
#endif

namespace wf {
namespace {

// Threads per sweep workgroup.  Workgroups that find their chunk skipped still
// cost a dispatch each, so this schedule uses fewer, larger workgroups than the
// full sweep, each issuing whole batches of loads.  Same-process A/B on 256
// chains of K = 16 at an 80% match rate (median of 5 trials, whole verify
// call): 512 threads 83.0 us; 256 threads 93.7 us; 1024 threads 94.9 us; the
// full sweep's loop form at 256 / 512 threads 99.8 / 102.6 us.
constexpr int kEeThreads = WF_EARLY_EXIT_THREADS;
// Sweep workgroups resident at once on the 256 compute units (32 waves each).
constexpr int64_t kEeResident = 256 * (32 * 64 / kEeThreads);

__global__ __launch_bounds__(kThreads) void early_exit_clear_kernel(int* __restrict__ flags, int B) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < B) flags[i] = 0;
}

template <int DT>
__global__ __launch_bounds__(kEeThreads) void early_exit_sweep_kernel(
    const unsigned char* __restrict__ logits, int64_t row_bytes, int V, int B, int K, int splits,
    int chunk_vecs, int nvec, const int32_t* __restrict__ draft, int* __restrict__ flags,
    Partial* __restrict__ part) {
  using E = Elem<DT>;
  const int per_pos = B * splits;
  const int pos = blockIdx.x / per_pos;
  const int rem = blockIdx.x - pos * per_pos;
  const int b = rem / splits;
  const int c = rem - b * splits;
  const int row = b * (K + 1) + pos;
  const int blk = row * splits + c;
  const unsigned char* rowp = logits + static_cast<int64_t>(row) * row_bytes;
  __shared__ int skip_s;
  // The flag and the draft token are loaded together.  The draft token's logit
  // is requested after the barrier (which waits for outstanding loads), so it
  // arrives during the sweep.
  int dtok = -1;
  if (threadIdx.x == 0) {
    const int e = pos > 0 ? __hip_atomic_load(&flags[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0;
    dtok = pos < K ? draft[static_cast<int64_t>(b) * K + pos] : -1;
    const bool skip = e > 0 && INT_MAX - e < pos;
    // A token outside the vocabulary never equals the greedy token.
    if (!skip && pos < K && (dtok < 0 || dtok >= V) && c == 0)
      __hip_atomic_fetch_max(&flags[b], INT_MAX - pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    skip_s = skip;
  }
  __syncthreads();
  if (skip_s) {
    if (threadIdx.x == 0) part[blk] = Partial{-INFINITY, INT_MAX};
    return;
  }
  const bool check = threadIdx.x == 0 && pos < K && dtok >= 0 && dtok < V;
  const float xd = check ? E::scalar(rowp, dtok) : 0.0f;
  const Partial r =
      sweep_chunk<DT, kEeThreads, true>(blk, logits, row_bytes, V, splits, chunk_vecs, nvec, part);
  if (check && (r.val > xd || (r.val == xd && r.idx < dtok)))
    __hip_atomic_fetch_max(&flags[b], INT_MAX - pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per sequence: merge the partials of every row (rows after n may
// be incomplete; only rows 0..n are used), scan for the first mismatch, and
// emit AL, the bonus token and row_argmax with -1 after n.
__global__ __launch_bounds__(kThreads) void early_exit_accept_kernel(
    const Partial* __restrict__ part, int splits, int K, const int32_t* __restrict__ draft,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus, int32_t* __restrict__ row_argmax) {
  __shared__ int t_s[kMaxSeqRows];
  __shared__ int n_s;
  const int b = blockIdx.x;
  const int R = K + 1;
  const int32_t* dr = draft + static_cast<int64_t>(b) * K;
  const int draft0 = K > 0 ? chain_load(dr, K) : -1;
  MergeIn mi;
  merge_load(mi, part, splits, b * R, R);
  merge_finish(mi, part, splits, b * R, R, t_s, nullptr);
  __syncthreads();
  chain_accept(draft0, t_s, K, dr, accept_len + b, bonus + b, &n_s);
  if (!row_argmax) return;
  __syncthreads();
  const int n = n_s;
  for (int i = threadIdx.x; i < R; i += kThreads)
    row_argmax[static_cast<int64_t>(b) * R + i] = i <= n ? t_s[i] : -1;
}

}  // namespace

SweepPlan early_exit_plan(int32_t B, int32_t V) {
  // Chunks of about one batch of 16-byte loads per thread (kEeThreads x 8
  // vectors of 8 bf16, 5 chunks per 151,936-wide row), starting on
  // 256-element boundaries.  Measured on 256 chains of K = 16 (whole call):
  // 4 / 5 / 8 / 10 chunks per row 87.2 / 82.6 / 95.8 / 105.2 us.  Small
  // batches are split further so that one position has at least as many
  // workgroups as are resident at once: then a sequence's next row is
  // dispatched only after its current row's workgroups have mostly finished,
  // and a mismatch found there is seen.  Chunks stay at least 2048 elements.
  const int64_t target = WF_EARLY_EXIT_CHUNK;
  int64_t splits = (V + target - 1) / target;
  const int64_t for_window = (kEeResident + B - 1) / (B > 0 ? B : 1);
  if (splits < for_window) splits = for_window;
  const int64_t max_splits = V / 2048 > 1 ? V / 2048 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t chunk = (V + splits - 1) / splits;
  chunk = (chunk + 255) / 256 * 256;
  splits = (V + chunk - 1) / chunk;
  return SweepPlan{static_cast<int32_t>(splits), static_cast<int32_t>(chunk)};
}

hipError_t launch_early_exit_chain(const void* logits, int dtype, int64_t row_stride, int32_t B,
                                   int32_t K, int32_t V, SweepPlan plan, const int32_t* draft,
                                   int* flags, Partial* part, int32_t* accept_len, int32_t* bonus,
                                   int32_t* row_argmax, hipStream_t stream) {
  hipLaunchKernelGGL(early_exit_clear_kernel, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, flags, B);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(B) * (K + 1) * plan.splits);
  const unsigned char* base = static_cast<const unsigned char*>(logits);
  if (dtype == WF_BF16) {
    using E = Elem<WF_BF16>;
    hipLaunchKernelGGL(early_exit_sweep_kernel<WF_BF16>, dim3(blocks), dim3(kEeThreads), 0, stream,
                       base, row_stride * E::kBytes, V, B, K, plan.splits, plan.chunk / E::kPerVec,
                       V / E::kPerVec, draft, flags, part);
  } else {
    using E = Elem<WF_F32>;
    hipLaunchKernelGGL(early_exit_sweep_kernel<WF_F32>, dim3(blocks), dim3(kEeThreads), 0, stream,
                       base, row_stride * E::kBytes, V, B, K, plan.splits, plan.chunk / E::kPerVec,
                       V / E::kPerVec, draft, flags, part);
  }
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(early_exit_accept_kernel, dim3(B), dim3(kThreads), 0, stream, part,
                     plan.splits, K, draft, accept_len, bonus, row_argmax);
  return hipGetLastError();
}

}  // namespace wf
