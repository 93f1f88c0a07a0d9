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
#include "common.h"

namespace wf {
namespace {

__device__ inline void take_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// t_s[i] = argmax of row (row0 + i) for i < nrows; row_argmax[row0 + i] too when given.
// A group of G lanes (the power of two >= splits, at most 64) merges one row, so
// a pass over the workgroup covers 256 / G rows with all their loads in flight.
__device__ void merge_rows(const Partial* __restrict__ part, int splits, int row0, int nrows,
                           int* t_s, int* __restrict__ row_argmax) {
  int G = 1;
  while (G < splits && G < 64) G <<= 1;
  const int per_pass = kThreads / G;
  const int sl = threadIdx.x & (G - 1);
  for (int base = 0; base < nrows; base += per_pass) {
    const int i = base + threadIdx.x / G;
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (i < nrows) {
      const Partial* p = part + static_cast<int64_t>(row0 + i) * splits;
      for (int s = sl; s < splits; s += G) take_better(bv, bi, p[s].val, p[s].idx);
    }
    for (int off = G >> 1; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      take_better(bv, bi, ov, oi);
    }
    if (sl == 0 && i < nrows) {
      if (i < kMaxSeqRows) t_s[i] = bi;
      if (row_argmax) row_argmax[row0 + i] = bi;
    }
  }
}

// Chain acceptance by wave 0: n = first i < K with draft[i] != t[i], else K.
__device__ void chain_accept(const int* t_s, int K, const int32_t* __restrict__ draft,
                             int32_t* al_out, int32_t* bonus_out, int32_t* best_out) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int n = K;
  for (int i0 = 0; i0 < K; i0 += 64) {
    const int i = i0 + lane;
    const bool mismatch = i < K && draft[i] != t_s[i];
    const unsigned long long mask = __ballot(mismatch);
    if (mask) {
      n = i0 + __ffsll(mask) - 1;
      break;
    }
  }
  if (lane == 0) {
    *al_out = n + 1;
    *bonus_out = t_s[n];
    if (best_out) *best_out = n;
  }
}

// Tree acceptance by the whole workgroup.  anc/dep/ok are LDS scratch of kMaxSeqRows.
__device__ void tree_accept(const int* t_s, int N, int V, const int32_t* __restrict__ parent,
                            const int32_t* __restrict__ draft_ids, const int32_t* __restrict__ d2t,
                            int Vd, int* anc, int* dep, int* ok, int* red, int32_t* al_out,
                            int32_t* bonus_out, int32_t* best_out) {
  const int tid = threadIdx.x;
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int u = tid + k * kThreads;
    if (u >= N) break;
    if (u == 0) {
      anc[0] = 0;
      dep[0] = 0;
      ok[0] = 1;
    } else {
      const int p = parent[u];
      const bool valid = p >= 0 && p < u;
      const int did = draft_ids[u];
      const int tok = (did >= 0 && did < Vd) ? d2t[did] : -1;
      const bool match = valid && tok >= 0 && tok < V && tok == t_s[valid ? p : 0];
      anc[u] = valid ? p : 0;
      dep[u] = 1;
      ok[u] = match ? 1 : 0;
    }
  }
  __syncthreads();
  // Pointer jumping: after r rounds anc[u] is u's 2^r-th ancestor (or the root),
  // dep[u] the number of edges to it, ok[u] the AND of the match bits on the way.
  for (int span = 1; span < N; span <<= 1) {
    int na[kRowsPerThread], nd[kRowsPerThread], no[kRowsPerThread];
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
      const int u = tid + k * kThreads;
      if (u < N) {
        const int a = anc[u];
        na[k] = anc[a];
        nd[k] = dep[u] + dep[a];
        no[k] = ok[u] & ok[a];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
      const int u = tid + k * kThreads;
      if (u < N) {
        anc[u] = na[k];
        dep[u] = nd[k];
        ok[u] = no[k];
      }
    }
    __syncthreads();
  }
  // Deepest accepted node, lowest index among equals: max of depth * 2^16 + (65535 - u).
  int key = -1;
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int u = tid + k * kThreads;
    if (u < N && ok[u]) key = max(key, (dep[u] << 16) | (0xffff - u));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off));
  if ((tid & 63) == 0) red[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    int k = red[0];
    for (int w = 1; w < kWaves; ++w) k = max(k, red[w]);
    const int best = 0xffff - (k & 0xffff);
    *al_out = (k >> 16) + 1;
    *bonus_out = t_s[best];
    if (best_out) *best_out = best;
  }
}

__global__ __launch_bounds__(kThreads) void finalize_chain_kernel(
    const Partial* __restrict__ part, int splits, int K, const int32_t* __restrict__ draft,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus, int32_t* __restrict__ row_argmax) {
  __shared__ int t_s[kMaxSeqRows];
  const int b = blockIdx.x;
  const int R = K + 1;
  merge_rows(part, splits, b * R, R, t_s, row_argmax);
  __syncthreads();
  chain_accept(t_s, K, draft + static_cast<int64_t>(b) * K, accept_len + b, bonus + b, nullptr);
}

__global__ __launch_bounds__(kThreads) void finalize_tree_kernel(
    const Partial* __restrict__ part, int splits, int N, int V, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ draft_ids, const int32_t* __restrict__ d2t, int Vd,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus, int32_t* __restrict__ best_node,
    int32_t* __restrict__ row_argmax) {
  __shared__ int t_s[kMaxSeqRows], anc[kMaxSeqRows], dep[kMaxSeqRows], ok[kMaxSeqRows];
  __shared__ int red[kWaves];
  const int b = blockIdx.x;
  merge_rows(part, splits, b * N, N, t_s, row_argmax);
  __syncthreads();
  const int64_t o = static_cast<int64_t>(b) * N;
  tree_accept(t_s, N, V, parent + o, draft_ids + o, d2t, Vd, anc, dep, ok, red, accept_len + b,
              bonus + b, best_node ? best_node + b : nullptr);
}

__global__ __launch_bounds__(kThreads) void finalize_routed_kernel(
    const Partial* __restrict__ part, int splits, int V, const int32_t* __restrict__ row_offsets,
    int total_rows, const int32_t* __restrict__ choice, int K, const int32_t* __restrict__ chain_draft,
    int N, const int32_t* __restrict__ parent, const int32_t* __restrict__ draft_ids,
    const int32_t* __restrict__ d2t, int Vd, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ bonus, int32_t* __restrict__ best_node, int32_t* __restrict__ row_argmax) {
  __shared__ int t_s[kMaxSeqRows], anc[kMaxSeqRows], dep[kMaxSeqRows], ok[kMaxSeqRows];
  __shared__ int red[kWaves];
  const int b = blockIdx.x;
  const int lo = row_offsets[b], hi = row_offsets[b + 1], c = choice[b];
  const bool in_range = lo >= 0 && lo <= hi && hi <= total_rows;
  const int rows = hi - lo;
  const bool chain = in_range && c == 0 && rows == K + 1;
  const bool tree = in_range && c == 1 && rows == N;
  if (in_range) merge_rows(part, splits, lo, rows, t_s, row_argmax);
  if (!chain && !tree) {
    if (threadIdx.x == 0) {
      accept_len[b] = 0;
      bonus[b] = -1;
      if (best_node) best_node[b] = -1;
    }
    return;
  }
  __syncthreads();
  if (chain) {
    chain_accept(t_s, K, chain_draft + static_cast<int64_t>(b) * K, accept_len + b, bonus + b,
                 best_node ? best_node + b : nullptr);
  } else {
    const int64_t o = static_cast<int64_t>(b) * N;
    tree_accept(t_s, N, V, parent + o, draft_ids + o, d2t, Vd, anc, dep, ok, red, accept_len + b,
                bonus + b, best_node ? best_node + b : nullptr);
  }
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

hipError_t launch_finalize_routed(const Partial* part, int32_t splits, int32_t B, int32_t V,
                                  const int32_t* row_offsets, int32_t total_rows,
                                  const int32_t* choice, int32_t K, const int32_t* chain_draft,
                                  int32_t N, const int32_t* parent, const int32_t* draft_ids,
                                  const int32_t* d2t, int32_t Vd, int32_t* accept_len,
                                  int32_t* bonus, int32_t* best_node, int32_t* row_argmax,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(finalize_routed_kernel, dim3(B), dim3(kThreads), 0, stream, part, splits, V,
                     row_offsets, total_rows, choice, K, chain_draft, N, parent, draft_ids, d2t, Vd,
                     accept_len, bonus, best_node, row_argmax);
  return hipGetLastError();
}

}  // namespace wf
