// Device building blocks of the per-sequence acceptance (WhiFlash paper,
// section 3.2): merging chunk partials into each row's greedy token, the DFlash
// chain scan and the EAGLE-3 tree propagation.  Used by the finalize kernels.
//
// The acceptance of one sequence is a short chain of dependent memory reads
// (row offsets -> chunk partials; draft ids -> d2t entries), so every piece
// is split into a load phase and a compute phase: a kernel first issues all
// loads that depend on nothing (offsets, choices, draft tokens, parents, draft
// ids), then all loads that depend on those (chunk partials, d2t entries), and
// only then reduces and propagates in registers and LDS.
#pragma once

#include "common.h"
#include "dpp.h"

namespace wf {

__device__ inline void better_partial(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// ---------------------------------------------------------------- row merge

// A group of G lanes (a power of two, about a quarter of the chunk count, at
// most 64) merges one row; each lane folds up to kMergePer partials.  The first
// pass over the workgroup (256 / G rows) is prefetched into registers.
constexpr int kMergePer = 4;

struct MergeIn {
  Partial q[kMergePer];
};

__device__ inline int merge_group(int splits) {
  int G = 1;
  while (G * kMergePer < splits && G < 64) G <<= 1;
  return G;
}

__device__ inline void merge_load(MergeIn& in, const Partial* __restrict__ part, int splits, int row0,
                                  int nrows) {
  const int G = merge_group(splits);
  const int i = threadIdx.x / G, sl = threadIdx.x & (G - 1);
  const Partial* p = part + static_cast<int64_t>(row0 + i) * splits;
#pragma unroll
  for (int u = 0; u < kMergePer; ++u) {
    const int s = sl + u * G;
    in.q[u] = (i < nrows && s < splits) ? p[s] : Partial{-INFINITY, INT_MAX};
  }
}

// t_s[i] = argmax of row (row0 + i) for i < nrows (i < kMaxSeqRows); row_argmax[row0 + i]
// too when given.  `in` holds the first pass; later passes and partials beyond
// G * kMergePer (only when splits > 256) are read here.
__device__ inline void merge_finish(const MergeIn& in, const Partial* __restrict__ part, int splits,
                                    int row0, int nrows, int* t_s, int* __restrict__ row_argmax) {
  const int G = merge_group(splits);
  const int per_pass = kThreads / G;
  const int sl = threadIdx.x & (G - 1);
  for (int base = 0; base < nrows; base += per_pass) {
    const int i = base + threadIdx.x / G;
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (i < nrows) {
      const Partial* p = part + static_cast<int64_t>(row0 + i) * splits;
      int s0 = sl;
      if (base == 0) {
#pragma unroll
        for (int u = 0; u < kMergePer; ++u) better_partial(bv, bi, in.q[u].val, in.q[u].idx);
        s0 += G * kMergePer;
      }
      for (; s0 < splits; s0 += G * kMergePer) {
        Partial q[kMergePer];
#pragma unroll
        for (int u = 0; u < kMergePer; ++u) {
          const int s = s0 + u * G;
          q[u] = s < splits ? p[s] : Partial{-INFINITY, INT_MAX};
        }
#pragma unroll
        for (int u = 0; u < kMergePer; ++u) better_partial(bv, bi, q[u].val, q[u].idx);
      }
    }
    // G is uniform, so these branches are too.  Groups of up to 16 lanes use
    // DPP moves (quads, then half rows, then rows); wider groups finish with
    // shuffles.  Every lane of a group ends with the group's winner.
    if (G >= 2) dpp_better<kDppQuadXor1>(bv, bi);
    if (G >= 4) dpp_better<kDppQuadXor2>(bv, bi);
    if (G >= 8) dpp_better<kDppHalfMirror>(bv, bi);
    if (G >= 16) dpp_better<kDppMirror>(bv, bi);
    for (int off = 16; off < G; off <<= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      better_partial(bv, bi, ov, oi);
    }
    if (sl == 0 && i < nrows) {
      if (i < kMaxSeqRows) t_s[i] = bi;
      if (row_argmax) row_argmax[row0 + i] = bi;
    }
  }
}

// ---------------------------------------------------------------- chain

// Draft tokens of the first 64 positions, one per lane of wave 0.
__device__ inline int chain_load(const int32_t* __restrict__ draft, int K) {
  const int lane = threadIdx.x;
  return (lane < 64 && lane < K) ? draft[lane] : -1;
}

// Chain acceptance by wave 0: n = first i < K with draft[i] != t[i], else K.
__device__ inline void chain_accept(int draft0, const int* t_s, int K,
                                    const int32_t* __restrict__ draft, int32_t* al_out,
                                    int32_t* bonus_out, int32_t* best_out) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int n = K;
  for (int i0 = 0; i0 < K; i0 += 64) {
    const int i = i0 + lane;
    const int d = i0 == 0 ? draft0 : (i < K ? draft[i] : -1);
    const bool mismatch = i < K && d != t_s[i];
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

// ---------------------------------------------------------------- tree

// Per-thread node inputs of one tree: node u = threadIdx.x + k * 256.
struct TreeIn {
  int p[kRowsPerThread];    // parent
  int tok[kRowsPerThread];  // draft id after tree_load_ids, target id after tree_load_tokens
};

__device__ inline void tree_load_ids(TreeIn& in, int N, const int32_t* __restrict__ parent,
                                     const int32_t* __restrict__ draft_ids) {
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int u = threadIdx.x + k * kThreads;
    const bool node = u >= 1 && u < N;
    in.p[k] = node ? parent[u] : -1;
    in.tok[k] = node ? draft_ids[u] : -1;
  }
}

// Draft ids outside [0, Vd) and table entries outside [0, V) become -1 (never match).
__device__ inline void tree_load_tokens(TreeIn& in, const int32_t* __restrict__ d2t, int Vd, int V) {
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int did = in.tok[k];
    const int tok = (did >= 0 && did < Vd) ? d2t[did] : -1;
    in.tok[k] = (tok >= 0 && tok < V) ? tok : -1;
  }
}

// Tree acceptance by the whole workgroup.  anc/dep/ok are LDS scratch of kMaxSeqRows.
// Node u >= 1 matches iff 0 <= parent < u and its target id equals t[parent];
// pointer jumping then gives every node the AND of the match bits on its root
// path and its depth in ceil(log2 N) rounds.
__device__ inline void tree_accept(const TreeIn& in, const int* t_s, int N, int* anc, int* dep, int* ok,
                                   int* red, int32_t* al_out, int32_t* bonus_out, int32_t* best_out) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int u = tid + k * kThreads;
    if (u < N) {
      if (u == 0) {
        anc[0] = 0;
        dep[0] = 0;
        ok[0] = 1;
      } else {
        const int p = in.p[k];
        const bool valid = p >= 0 && p < u;
        const int tok = in.tok[k];
        const bool match = valid && tok >= 0 && tok == t_s[valid ? p : 0];
        anc[u] = valid ? p : 0;
        dep[u] = 1;
        ok[u] = match ? 1 : 0;
      }
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
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int u = tid + k * kThreads;
    if (u < N && ok[u]) key = max(key, (dep[u] << 16) | (0xffff - u));
  }
  key = wave_max_to_lane63(key);
  if ((tid & 63) == 63) red[tid >> 6] = key;
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

// ---------------------------------------------------------------- routed

// LDS used by one sequence's acceptance.
struct AcceptLds {
  int t_s[kMaxSeqRows], anc[kMaxSeqRows], dep[kMaxSeqRows], ok[kMaxSeqRows];
  int red[kWaves];
  int best;
};

// Arguments of the routed dispatch (see whiflash_verify_routed).
struct RoutedArgs {
  const Partial* part;
  int splits, V;
  const int32_t* row_offsets;
  int total_rows, K;
  const int32_t* chain_draft;
  int N;
  const int32_t* parent;
  const int32_t* draft_ids;
  const int32_t* d2t;
  int Vd;
  int32_t* accept_len;
  int32_t* bonus;
  int32_t* best_node;
  int32_t* row_argmax;
  // Early-exit schedule: only the rows of accepted nodes were read whole, so
  // row_argmax gets t for those rows and -1 for the others.
  bool early = false;
};

// Loads of sequence b of a routed batch that depend on nothing else.  The
// chain and tree inputs are both read (a few hundred bytes), so the drafter
// choice is not needed before the second phase.
struct RoutedIn {
  int lo, hi;
  int draft0;
  TreeIn tree;
  MergeIn merge;
};

__device__ inline void routed_load_phase1(RoutedIn& in, const RoutedArgs& a, int b) {
  in.lo = a.row_offsets[b];
  in.hi = a.row_offsets[b + 1];
  in.draft0 = a.K > 0 ? chain_load(a.chain_draft + static_cast<int64_t>(b) * a.K, a.K) : -1;
  const int64_t o = static_cast<int64_t>(b) * a.N;
  tree_load_ids(in.tree, a.N, a.parent + o, a.draft_ids + o);
}

__device__ inline bool routed_in_range(const RoutedIn& in, const RoutedArgs& a) {
  return in.lo >= 0 && in.lo <= in.hi && in.hi <= a.total_rows;
}

__device__ inline void routed_load_phase2(RoutedIn& in, const RoutedArgs& a) {
  if (routed_in_range(in, a)) merge_load(in.merge, a.part, a.splits, in.lo, in.hi - in.lo);
  tree_load_tokens(in.tree, a.d2t, a.Vd, a.V);
}

// Sequence b verified with drafter choice c by the whole workgroup: chain rows
// for c == 0, tree rows for c == 1, else malformed.
__device__ inline void routed_accept(const RoutedIn& in, const RoutedArgs& a, int b, int c,
                                     AcceptLds& L) {
  const bool in_range = routed_in_range(in, a);
  const int rows = in.hi - in.lo;
  const bool chain = in_range && c == 0 && rows == a.K + 1;
  const bool tree = in_range && c == 1 && rows == a.N;
  if (in_range)
    merge_finish(in.merge, a.part, a.splits, in.lo, rows, L.t_s, a.early ? nullptr : a.row_argmax);
  if (!chain && !tree) {
    if (threadIdx.x == 0) {
      a.accept_len[b] = 0;
      a.bonus[b] = -1;
      if (a.best_node) a.best_node[b] = -1;
    }
    if (a.early && a.row_argmax && in_range)
      for (int i = threadIdx.x; i < rows; i += kThreads) a.row_argmax[in.lo + i] = -1;
    return;
  }
  __syncthreads();
  int32_t* best_out = a.early ? &L.best : (a.best_node ? a.best_node + b : nullptr);
  if (chain) {
    chain_accept(in.draft0, L.t_s, a.K, a.chain_draft + static_cast<int64_t>(b) * a.K,
                 a.accept_len + b, a.bonus + b, best_out);
  } else {
    tree_accept(in.tree, L.t_s, a.N, L.anc, L.dep, L.ok, L.red, a.accept_len + b, a.bonus + b,
                best_out);
  }
  if (!a.early) return;
  __syncthreads();
  const int best = L.best;
  if (threadIdx.x == 0 && a.best_node) a.best_node[b] = best;
  if (a.row_argmax) {
    for (int i = threadIdx.x; i < rows; i += kThreads) {
      const bool accepted = chain ? i <= best : L.ok[i] != 0;
      a.row_argmax[in.lo + i] = accepted ? L.t_s[i] : -1;
    }
  }
}

}  // namespace wf
