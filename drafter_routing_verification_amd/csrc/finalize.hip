// Per-sequence acceptance after the argmax sweep: merge the chunk partials of
// each row into the target token t, then
//   chain (DFlash block; WhiFlash paper, section 3.2): first mismatch via a
//     wave ballot, AL = n + 1, bonus = t[n];
//   tree (EAGLE-3 draft tree; same section, d2t map from the Qwen3-4B-EAGLE3
//     card): every node's match bit is computed in parallel, then pointer
//     jumping in LDS gives each node the AND of the match bits and the length
//     of its root path in ceil(log2 N) rounds; the deepest accepted node
//     (lowest index on ties) is a block-wide max of (depth, -index);
//   routed: per-sequence dispatch over ragged packed rows, with a defined
//     result (AL 0, bonus -1) for malformed sequences.
// One 256-thread workgroup per sequence; rows of a sequence live in LDS.
#include "accept.h"
#include "common.h"

namespace wf {
namespace {

__global__ __launch_bounds__(kThreads) void finalize_chain_kernel(
    const Partial* __restrict__ part, int splits, int K, const int32_t* __restrict__ draft,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus, int32_t* __restrict__ row_argmax) {
  __shared__ int t_s[kMaxSeqRows];
  const int b = blockIdx.x;
  const int R = K + 1;
  const int32_t* dr = draft + static_cast<int64_t>(b) * K;
  const int draft0 = K > 0 ? chain_load(dr, K) : -1;
  MergeIn mi;
  merge_load(mi, part, splits, b * R, R);
  merge_finish(mi, part, splits, b * R, R, t_s, row_argmax);
  __syncthreads();
  chain_accept(draft0, t_s, K, dr, accept_len + b, bonus + b, nullptr);
}

__global__ __launch_bounds__(kThreads) void finalize_tree_kernel(
    const Partial* __restrict__ part, int splits, int N, int V, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ draft_ids, const int32_t* __restrict__ d2t, int Vd,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus, int32_t* __restrict__ best_node,
    int32_t* __restrict__ row_argmax) {
  __shared__ AcceptLds L;
  const int b = blockIdx.x;
  const int64_t o = static_cast<int64_t>(b) * N;
  TreeIn ti;
  tree_load_ids(ti, N, parent + o, draft_ids + o);
  MergeIn mi;
  merge_load(mi, part, splits, b * N, N);
  tree_load_tokens(ti, d2t, Vd, V);
  merge_finish(mi, part, splits, b * N, N, L.t_s, row_argmax);
  __syncthreads();
  tree_accept(ti, L.t_s, N, L.anc, L.dep, L.ok, L.red, accept_len + b, bonus + b,
              best_node ? best_node + b : nullptr);
}

__global__ __launch_bounds__(kThreads) void finalize_routed_kernel(RoutedArgs args,
                                                                   const int32_t* __restrict__ choice) {
  __shared__ AcceptLds lds;
  const int b = blockIdx.x;
  RoutedIn in;
  routed_load_phase1(in, args, b);
  const int c = choice[b];
  routed_load_phase2(in, args);
  routed_accept(in, args, b, c, lds);
}

}  // namespace

hipError_t launch_finalize_chain(const Partial* part, int32_t splits, int32_t B, int32_t K,
                                 const int32_t* draft, int32_t* accept_len, int32_t* bonus,
                                 int32_t* row_argmax, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_chain_kernel, dim3(B), dim3(kThreads), 0, stream, part, splits, K,
                     draft, accept_len, bonus, row_argmax);
  return hipGetLastError();
}

hipError_t launch_finalize_tree(const Partial* part, int32_t splits, int32_t B, int32_t N, int32_t V,
                                const int32_t* parent, const int32_t* draft_ids, const int32_t* d2t,
                                int32_t Vd, int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                                int32_t* row_argmax, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_tree_kernel, dim3(B), dim3(kThreads), 0, stream, part, splits, N, V,
                     parent, draft_ids, d2t, Vd, accept_len, bonus, best_node, row_argmax);
  return hipGetLastError();
}

hipError_t launch_finalize_routed(bool early, const Partial* part, int32_t splits, int32_t B, int32_t V,
                                  const int32_t* row_offsets, int32_t total_rows,
                                  const int32_t* choice, int32_t K, const int32_t* chain_draft,
                                  int32_t N, const int32_t* parent, const int32_t* draft_ids,
                                  const int32_t* d2t, int32_t Vd, int32_t* accept_len,
                                  int32_t* bonus, int32_t* best_node, int32_t* row_argmax,
                                  hipStream_t stream) {
  const RoutedArgs args{part,      splits, V,  row_offsets, total_rows, K,
                        chain_draft, N,     parent, draft_ids, d2t,   Vd,
                        accept_len, bonus,  best_node, row_argmax, early};
  hipLaunchKernelGGL(finalize_routed_kernel, dim3(B), dim3(kThreads), 0, stream, args, choice);
  return hipGetLastError();
}

}  // namespace wf
