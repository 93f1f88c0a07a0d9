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
//
// Trees and routed batches.  An EAGLE-3 draft tree needs only the rows of its
// accepted nodes: node u >= 1 is accepted iff its parent p is accepted and its
// target token equals t[p] (same section: a tree of candidate tokens is
// verified), and the bonus token is t[best].  A DFlash chain is the tree whose
// node i + 1 hangs under node i with token draft[i], so one schedule serves
// both and the routed mix.  A per-sequence prep kernel writes, for every node,
// its ancestor-or-self bit mask and its edge (parent, target token, and the
// parent row's logit at that token), and starts each sequence's rejected-node
// mask with the nodes that can never match.  The sweep launches node-major
// (every sequence's node 0, then node 1, ...; parents precede children since
// parent[u] < u).  A chunk is skipped when its node's ancestor mask meets the
// rejected mask; a chunk whose maximum beats a child's (logit, token) marks
// that child rejected with an agent-scope atomic or.  Marks only name nodes
// that are truly not accepted, so accepted rows are always read whole.
// Skipped chunks write nothing: routed row ranges may overlap, and a row one
// sequence skips may be read by another.  The routed acceptance then runs on
// the merged partials as in the full path (rows of nodes that are not
// accepted never decide anything) and reports -1 for them in row_argmax.
#include "accept.h"
#include "common.h"
#include "router_math.h"
#include "sweep_body.h"

#ifndef WF_EARLY_EXIT_THREADS
#define WF_EARLY_EXIT_THREADS 512
#endif
#ifndef WF_EARLY_EXIT_CHUNK
#define WF_EARLY_EXIT_CHUNK 51200
#endif
#ifndef WF_EE_TREE_GROUP_FROM
#define WF_EE_TREE_GROUP_FROM 10
#endif
#ifndef WF_EE_TREE_GROUP
#define WF_EE_TREE_GROUP 8
#endif

namespace wf {
namespace {

// Threads per sweep workgroup.  Workgroups that find their chunk skipped still
// cost a dispatch each, so this schedule uses fewer, larger workgroups than the
// full sweep, each issuing whole batches of loads.  Same-process A/B on 256
// chains of K = 16 at an 80% match rate, 5 chunks per row (median of 5
// trials, whole verify call): 512 threads 83.0 us; 256 threads 93.7 us; 1024
// threads 94.9 us; the full sweep's loop form at 256 / 512 threads 99.8 /
// 102.6 us.
constexpr int kEeThreads = WF_EARLY_EXIT_THREADS;

// From node index kTreeGroupFrom on, one tree-sweep workgroup covers the same
// chunk of node u in kTreeGroup sequences: it reads their rows and masks in one
// round trip and sweeps only the chunks still needed, one after another.  High
// node indices are mostly absent (chains end at K) or rejected, so this saves
// the dispatch and the round trip of a workgroup per skipped chunk.
// Same-process A/B on the routed early-exit round (whole call, 64 chains of
// K = 16 and 64 trees of 61 nodes): one workgroup per (node, sequence, chunk)
// 82.8 us; (from, group) = (10, 8) 72.7 us; (10, 6) 72.9; (8, 8) 73.3;
// (12, 8) 73.2; (7, 6) 73.4; (12, 12) 74.6; (17, 8) 75.9; (17, 16) 75.3;
// (8, 4) 75.7; (6, 4) 76.1; (5, 8) 77.7; (24, 8) 77.8; (10, 32) 89.2.  The
// same grouping on the chain-only schedule was slower (its late positions
// still read about a third of their rows).
constexpr int kTreeGroupFrom = WF_EE_TREE_GROUP_FROM;
constexpr int kTreeGroup = WF_EE_TREE_GROUP;

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

// Early-exit chain round: the acceptance above plus the router's finish for
// sequence b (its choice is for the next round; the chain scan does not use it).
template <int DT>
__global__ __launch_bounds__(kThreads) void early_exit_round_accept_kernel(
    const float* __restrict__ zp, int KS, int B, int m, const float* __restrict__ b1,
    const void* __restrict__ W2, const float* __restrict__ b2, float tau,
    float* __restrict__ delta_al, int32_t* __restrict__ choice, const Partial* __restrict__ part,
    int splits, int K, const int32_t* __restrict__ draft, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ bonus, int32_t* __restrict__ row_argmax) {
  __shared__ int t_s[kMaxSeqRows];
  __shared__ int n_s;
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
  merge_finish(mi, part, splits, b * R, R, t_s, nullptr);
  const float dal = router_finish_compute<DT>(fin, zp, direct, KS, B, m, b, b1, W2, b2, redf);
  if (threadIdx.x == 0) {
    delta_al[b] = dal;
    choice[b] = dal > tau ? 1 : 0;
  }
  // router_finish_compute ends with a barrier, so t_s is complete here.
  chain_accept(draft0, t_s, K, dr, accept_len + b, bonus + b, &n_s);
  if (!row_argmax) return;
  __syncthreads();
  const int n = n_s;
  for (int i = threadIdx.x; i < R; i += kThreads)
    row_argmax[static_cast<int64_t>(b) * R + i] = i <= n ? t_s[i] : -1;
}

// ----------------------------------------------------------------- trees and routed batches

// Node table of one sequence (prep kernel, one 256-thread workgroup per
// sequence, c = its drafter choice).  p_s is LDS of kMaxSeqRows ints, mask_s
// LDS of kMaxMaskWords words.
__device__ inline void ee_prep_sequence(const EeTreeArgs& a, int b, int c, int* p_s,
                                        unsigned long long* mask_s) {
  const int tid = threadIdx.x;
  const int lo = a.row_offsets ? a.row_offsets[b] : b * a.N;
  const int hi = a.row_offsets ? a.row_offsets[b + 1] : lo + a.N;
  const bool in_range = lo >= 0 && lo <= hi && hi <= a.total_rows;
  const int n = hi - lo;
  const bool chain = in_range && c == 0 && n == a.K + 1;
  const bool tree = in_range && c == 1 && n == a.N;
  const bool ok = chain || tree;
  for (int u = tid; u < a.Rmax; u += kThreads)
    a.rowmap[static_cast<int64_t>(u) * a.B + b] = ok && u < n ? lo + u : -1;
  if (!ok) return;  // malformed: no row of this sequence is read
  for (int w = tid; w < a.W; w += kThreads) mask_s[w] = 0ull;
  __syncthreads();
  const unsigned char* base = a.logits + static_cast<int64_t>(lo) * a.row_bytes;
  for (int u = tid; u < a.Rmax; u += kThreads) {
    int p = -1, tok = -1;
    if (u >= 1 && u < n) {
      if (chain) {
        p = u - 1;
        tok = a.chain_draft[static_cast<int64_t>(b) * a.K + u - 1];
      } else {
        p = a.parent[static_cast<int64_t>(b) * a.N + u];
        const int did = a.draft_ids[static_cast<int64_t>(b) * a.N + u];
        tok = did >= 0 && did < a.Vd ? a.d2t[did] : -1;
      }
    }
    const bool reach = u >= 1 && u < n && p >= 0 && p < u;
    const bool valid = reach && tok >= 0 && tok < a.V;
    if (u < kMaxSeqRows) p_s[u] = reach ? p : -1;
    if (u >= 1 && u < n && !valid) atomicOr(&mask_s[u >> 6], 1ull << (u & 63));
    float xv = 0.0f;
    if (valid) {
      const unsigned char* rowp = base + static_cast<int64_t>(p) * a.row_bytes;
      xv = a.dtype == WF_BF16 ? Elem<WF_BF16>::scalar(rowp, tok) : Elem<WF_F32>::scalar(rowp, tok);
    }
    a.edge[static_cast<int64_t>(b) * a.Rmax + u] = make_int4(p, tok, __float_as_int(xv), valid ? 1 : 0);
  }
  __syncthreads();
  // Ancestor-or-self masks: a chain's node u has bits 0..u; a tree node walks
  // its parents (each strictly smaller, so the walk ends at the root or at an
  // unreachable node).
  for (int u = tid; u < n; u += kThreads) {
    for (int w = 0; w < a.W; ++w) {
      unsigned long long m = 0ull;
      if (chain) {
        const int lo_bit = w * 64;
        if (u >= lo_bit + 63) m = ~0ull;
        else if (u >= lo_bit) m = (2ull << (u - lo_bit)) - 1ull;
      } else {
        for (int v = u; v >= 0; v = p_s[v])
          if ((v >> 6) == w) m |= 1ull << (v & 63);
      }
      a.anc[(static_cast<int64_t>(b) * a.Rmax + u) * a.W + w] = m;
    }
  }
  for (int w = tid; w < a.W; w += kThreads) a.mask[static_cast<int64_t>(b) * a.W + w] = mask_s[w];
}

__global__ __launch_bounds__(kThreads) void ee_prep_kernel(EeTreeArgs a) {
  __shared__ int p_s[kMaxSeqRows];
  __shared__ unsigned long long mask_s[kMaxMaskWords];
  const int b = blockIdx.x;
  int c = 1;
  if (a.choice) {
    c = a.choice[b];
  } else if (threadIdx.x == 0) {  // tree-only batch: offsets and choices for the acceptance
    a.seq_off[b] = b * a.N;
    if (b == a.B - 1) a.seq_off[a.B] = a.B * a.N;
    a.seq_choice[b] = 1;
  }
  ee_prep_sequence(a, b, c, p_s, mask_s);
}

// Routed round: finish the router for sequence b (Delta-AL, choice), then
// prepare the sequence for the drafter it chose.
template <int DT>
__global__ __launch_bounds__(kThreads) void ee_round_prep_kernel(
    EeTreeArgs a, const float* __restrict__ zp, int KS, int m, const float* __restrict__ b1,
    const void* __restrict__ W2, const float* __restrict__ b2, float tau,
    float* __restrict__ delta_al, int32_t* __restrict__ choice) {
  __shared__ int p_s[kMaxSeqRows];
  __shared__ unsigned long long mask_s[kMaxMaskWords];
  __shared__ float redf[kWaves];
  const int b = blockIdx.x;
  const HiddenSel direct{nullptr, nullptr, 0, 0};
  FinishIn fin;
  finish_load_pass<DT>(fin, zp, KS, a.B, m, b, 0, b1, W2, b2, direct);
  const float dal = router_finish_compute<DT>(fin, zp, direct, KS, a.B, m, b, b1, W2, b2, redf);
  const int c = dal > tau ? 1 : 0;
  if (threadIdx.x == 0) {
    delta_al[b] = dal;
    choice[b] = c;
  }
  ee_prep_sequence(a, b, c, p_s, mask_s);
}

// Sweeps chunk c of row `row`, node u of sequence b, and marks the children of
// u that the chunk proves are not accepted.
template <int DT>
__device__ void ee_tree_read(const EeTreeArgs& a, int splits, int chunk_vecs, int nvec,
                             Partial* __restrict__ part, int u, int b, int c, int row) {
  __shared__ float bv_s;
  __shared__ int bi_s;
  const int tid = threadIdx.x;
  // Edges of this sequence (one per node), consumed after the sweep.  They are
  // loaded unconditionally (threads past Rmax read the last node's edge and
  // ignore it): guarded loads let the compiler test each edge as soon as it
  // arrived, which held the sweep back by two round trips.
  const int4* eb = a.edge + static_cast<int64_t>(b) * a.Rmax;
  const int4 e0 = eb[tid < a.Rmax ? tid : a.Rmax - 1];
  const int4 e1 = eb[tid + kEeThreads < a.Rmax ? tid + kEeThreads : a.Rmax - 1];
  const Partial r = sweep_chunk<DT, kEeThreads, true>(row * splits + c, a.logits, a.row_bytes, a.V,
                                                      splits, chunk_vecs, nvec, part);
  if (tid == 0) {
    bv_s = r.val;
    bi_s = r.idx;
  }
  __syncthreads();
  const float bv = bv_s;
  const int bi = bi_s;
  unsigned long long* mb = a.mask + static_cast<int64_t>(b) * a.W;
  // A child whose (logit, token) is beaten inside this chunk is not the greedy
  // token of this row, so it is not accepted.
  if (tid < a.Rmax && e0.w && e0.x == u) {
    const float xv = __int_as_float(e0.z);
    if (bv > xv || (bv == xv && bi < e0.y))
      __hip_atomic_fetch_or(&mb[tid >> 6], 1ull << (tid & 63), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid + kEeThreads < a.Rmax && e1.w && e1.x == u) {
    const int v = tid + kEeThreads;
    const float xv = __int_as_float(e1.z);
    if (bv > xv || (bv == xv && bi < e1.y))
      __hip_atomic_fetch_or(&mb[v >> 6], 1ull << (v & 63), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Chunk c of node u in sequences b0 .. b0 + nb - 1: one round trip reads every
// item's row and masks, then the items still needed are swept one after another.
template <int DT>
__device__ void ee_tree_group(const EeTreeArgs& a, int splits, int chunk_vecs, int nvec,
                              Partial* __restrict__ part, int u, int b0, int nb, int c) {
  __shared__ int grow_s[kTreeGroup];
  __shared__ int grej_s[kTreeGroup];
  static_assert(kTreeGroup * kMaxMaskWords <= kEeThreads, "one (sequence, mask word) per thread");
  const int tid = threadIdx.x;
  // Every item's row and mask words in one round of loads, issued
  // unconditionally (threads past the items read item 0 and ignore it).
  const int nw = nb * a.W;
  const int t = tid < nw ? tid : 0;
  const int j = t / a.W, w = t - j * a.W;
  const int row = a.rowmap[static_cast<int64_t>(u) * a.B + b0 + (tid < nb ? tid : 0)];
  const unsigned long long m = __hip_atomic_load(&a.mask[static_cast<int64_t>(b0 + j) * a.W + w],
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long an = a.anc[(static_cast<int64_t>(b0 + j) * a.Rmax + u) * a.W + w];
  if (tid < kTreeGroup) grej_s[tid] = 0;
  __syncthreads();
  if (tid < nb) grow_s[tid] = row;
  if (tid < nw && (m & an) != 0ull) grej_s[j] = 1;
  __syncthreads();
  for (int j = 0; j < nb; ++j) {
    const int row = grow_s[j];
    if (row < 0 || grej_s[j]) continue;  // no such node, or not accepted
    ee_tree_read<DT>(a, splits, chunk_vecs, nvec, part, u, b0 + j, c, row);
    __syncthreads();  // LDS of the sweep and of the edge test is reused by the next item
  }
}

template <int DT>
__global__ __launch_bounds__(kEeThreads) void ee_tree_sweep_kernel(EeTreeArgs a, int splits,
                                                                    int chunk_vecs, int nvec,
                                                                    Partial* __restrict__ part) {
  const int per_u = a.B * splits;
  const int single_u = a.Rmax < kTreeGroupFrom ? a.Rmax : kTreeGroupFrom;
  const int single_blocks = single_u * per_u;
  if (static_cast<int>(blockIdx.x) >= single_blocks) {
    const int groups = (a.B + kTreeGroup - 1) / kTreeGroup;
    const int lb = blockIdx.x - single_blocks;
    const int gu = single_u + lb / (groups * splits);
    const int grem = lb - (gu - single_u) * groups * splits;
    const int g = grem / splits;
    const int b0 = g * kTreeGroup;
    ee_tree_group<DT>(a, splits, chunk_vecs, nvec, part, gu, b0,
                      a.B - b0 < kTreeGroup ? a.B - b0 : kTreeGroup, grem - g * splits);
    return;
  }
  const int u = blockIdx.x / per_u;
  const int rem = blockIdx.x - u * per_u;
  const int b = rem / splits;
  const int c = rem - b * splits;
  __shared__ int row_s;
  const int tid = threadIdx.x;
  if (tid < 64) {
    // The row and the mask words are loaded together, unconditionally (lanes
    // past W read word 0 and ignore it), in one round trip.
    const int row = a.rowmap[static_cast<int64_t>(u) * a.B + b];
    const int w = tid < a.W ? tid : 0;
    const unsigned long long m = __hip_atomic_load(&a.mask[static_cast<int64_t>(b) * a.W + w],
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long an = a.anc[(static_cast<int64_t>(b) * a.Rmax + u) * a.W + w];
    const bool hit = tid < a.W && (m & an) != 0ull;
    const bool rejected = __ballot(hit) != 0ull;
    if (tid == 0) row_s = rejected ? -1 : row;
  }
  __syncthreads();
  const int row = row_s;
  if (row < 0) return;  // no such node, or not accepted: nothing is written
  ee_tree_read<DT>(a, splits, chunk_vecs, nvec, part, u, b, c, row);
}

}  // namespace

SweepPlan early_exit_plan(int32_t B, int32_t V) {
  // Chunks of ~51K elements (3 per 151,936-wide row), starting on 256-element
  // boundaries.  Every chunk of a skipped row still costs a dispatch and a
  // flag round trip, so few chunks per row pay; too few lengthen each row's
  // read on the chain of dependent rows.  Measured, whole call, on the routed
  // workload (128 sequences, 4,992 rows) / the chain workload (256 chains of
  // K = 16): 1 chunk per row 88.3 / 112.9 us, 2 chunks 72.1 / 87.1 us,
  // 3 chunks 72.1 / 83.2 us, 5 chunks 79.6 / 83.0 us, 8 chunks (one position's
  // workgroups filling the resident slots) 100.4 / 82.6 us, 12 chunks 126.3 /
  // 115.8 us; 1024-thread workgroups over 1 or 2 chunks 77.5-81.0 / 91.0-97.3.
  (void)B;
  constexpr int64_t kChunkTarget = WF_EARLY_EXIT_CHUNK;
  int64_t splits = (V + kChunkTarget - 1) / kChunkTarget;
  const int64_t max_splits = V / 2048 > 1 ? V / 2048 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t chunk = (V + splits - 1) / splits;
  chunk = (chunk + 255) / 256 * 256;
  splits = (V + chunk - 1) / chunk;
  return SweepPlan{static_cast<int32_t>(splits), static_cast<int32_t>(chunk)};
}

static hipError_t launch_early_exit_sweep(const void* logits, int dtype, int64_t row_stride,
                                          int32_t B, int32_t K, int32_t V, SweepPlan plan,
                                          const int32_t* draft, int* flags, Partial* part,
                                          hipStream_t stream) {
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
  return hipGetLastError();
}

hipError_t launch_early_exit_chain(const void* logits, int dtype, int64_t row_stride, int32_t B,
                                   int32_t K, int32_t V, SweepPlan plan, const int32_t* draft,
                                   int* flags, Partial* part, int32_t* accept_len, int32_t* bonus,
                                   int32_t* row_argmax, hipStream_t stream) {
  hipLaunchKernelGGL(early_exit_clear_kernel, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, flags, B);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (launch_early_exit_sweep(logits, dtype, row_stride, B, K, V, plan, draft, flags, part,
                              stream) != hipSuccess)
    return hipErrorLaunchFailure;
  hipLaunchKernelGGL(early_exit_accept_kernel, dim3(B), dim3(kThreads), 0, stream, part,
                     plan.splits, K, draft, accept_len, bonus, row_argmax);
  return hipGetLastError();
}

hipError_t launch_early_exit_round(const void* logits, int dtype, int64_t row_stride, int32_t B,
                                   int32_t K, int32_t V, SweepPlan plan, const int32_t* draft,
                                   int* flags, Partial* part, int hidden_dtype,
                                   const RouterPlan& rplan, const float* zp, int32_t m,
                                   const float* b1, const void* W2, const float* b2, float tau,
                                   float* delta_al, int32_t* choice, int32_t* accept_len,
                                   int32_t* bonus, int32_t* row_argmax, hipStream_t stream) {
  if (launch_early_exit_sweep(logits, dtype, row_stride, B, K, V, plan, draft, flags, part,
                              stream) != hipSuccess)
    return hipErrorLaunchFailure;
  if (hidden_dtype == WF_BF16)
    hipLaunchKernelGGL(early_exit_round_accept_kernel<WF_BF16>, dim3(B), dim3(kThreads), 0, stream,
                       zp, rplan.slices, B, m, b1, W2, b2, tau, delta_al, choice, part,
                       plan.splits, K, draft, accept_len, bonus, row_argmax);
  else
    hipLaunchKernelGGL(early_exit_round_accept_kernel<WF_F32>, dim3(B), dim3(kThreads), 0, stream,
                       zp, rplan.slices, B, m, b1, W2, b2, tau, delta_al, choice, part,
                       plan.splits, K, draft, accept_len, bonus, row_argmax);
  return hipGetLastError();
}

EeTreeWs ee_tree_workspace(int32_t B, int32_t Rmax, int32_t total_rows, int32_t V, size_t align) {
  auto up = [align](size_t x) { return (x + align - 1) / align * align; };
  EeTreeWs w{};
  const size_t W = static_cast<size_t>((Rmax + 63) / 64);
  const SweepPlan plan = early_exit_plan(B, V);
  w.mask = 0;
  w.anc = w.mask + up(static_cast<size_t>(B) * W * 8);
  w.rowmap = w.anc + up(static_cast<size_t>(B) * Rmax * W * 8);
  w.edge = w.rowmap + up(static_cast<size_t>(B) * Rmax * 4);
  w.seq_off = w.edge + up(static_cast<size_t>(B) * Rmax * 16);
  w.seq_choice = w.seq_off + up((static_cast<size_t>(B) + 1) * 4);
  w.part = w.seq_choice + up(static_cast<size_t>(B) * 4);
  w.total = w.part + up(static_cast<size_t>(total_rows) * plan.splits * sizeof(Partial));
  return w;
}

EeTreeArgs ee_tree_args(char* ws, const EeTreeWs& off, int32_t B, int32_t Rmax, const void* logits,
                        int dtype, int64_t row_stride, int32_t V, const int32_t* row_offsets,
                        const int32_t* choice, int32_t total_rows, int32_t K,
                        const int32_t* chain_draft, int32_t N, const int32_t* parent,
                        const int32_t* draft_ids, const int32_t* d2t, int32_t Vd) {
  EeTreeArgs a{};
  a.B = B;
  a.Rmax = Rmax;
  a.W = (Rmax + 63) / 64;
  a.row_offsets = row_offsets;
  a.choice = choice;
  a.total_rows = total_rows;
  a.K = K;
  a.N = N;
  a.V = V;
  a.Vd = Vd;
  a.chain_draft = chain_draft;
  a.parent = parent;
  a.draft_ids = draft_ids;
  a.d2t = d2t;
  a.logits = static_cast<const unsigned char*>(logits);
  a.row_bytes = row_stride * (dtype == WF_BF16 ? 2 : 4);
  a.dtype = dtype;
  a.mask = reinterpret_cast<unsigned long long*>(ws + off.mask);
  a.anc = reinterpret_cast<unsigned long long*>(ws + off.anc);
  a.rowmap = reinterpret_cast<int32_t*>(ws + off.rowmap);
  a.edge = reinterpret_cast<int4*>(ws + off.edge);
  a.seq_off = reinterpret_cast<int32_t*>(ws + off.seq_off);
  a.seq_choice = reinterpret_cast<int32_t*>(ws + off.seq_choice);
  return a;
}

hipError_t launch_ee_tree_prep(const EeTreeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(ee_prep_kernel, dim3(a.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ee_round_prep(const EeTreeArgs& a, int hidden_dtype, const RouterPlan& plan,
                                const float* zp, int32_t m, const float* b1, const void* W2,
                                const float* b2, float tau, float* delta_al, int32_t* choice,
                                hipStream_t stream) {
  if (hidden_dtype == WF_BF16)
    hipLaunchKernelGGL(ee_round_prep_kernel<WF_BF16>, dim3(a.B), dim3(kThreads), 0, stream, a, zp,
                       plan.slices, m, b1, W2, b2, tau, delta_al, choice);
  else
    hipLaunchKernelGGL(ee_round_prep_kernel<WF_F32>, dim3(a.B), dim3(kThreads), 0, stream, a, zp,
                       plan.slices, m, b1, W2, b2, tau, delta_al, choice);
  return hipGetLastError();
}

hipError_t launch_ee_tree_sweep(const EeTreeArgs& a, SweepPlan plan, Partial* part,
                                hipStream_t stream) {
  // Node indices before kTreeGroupFrom: one workgroup per (sequence, chunk);
  // later ones: one per (group of kTreeGroup sequences, chunk).
  const int64_t single_u = a.Rmax < kTreeGroupFrom ? a.Rmax : kTreeGroupFrom;
  const int64_t groups = (a.B + kTreeGroup - 1) / kTreeGroup;
  const unsigned blocks = static_cast<unsigned>(
      (single_u * a.B + (a.Rmax - single_u) * groups) * plan.splits);
  if (a.dtype == WF_BF16) {
    using E = Elem<WF_BF16>;
    hipLaunchKernelGGL(ee_tree_sweep_kernel<WF_BF16>, dim3(blocks), dim3(kEeThreads), 0, stream, a,
                       plan.splits, plan.chunk / E::kPerVec, a.V / E::kPerVec, part);
  } else {
    using E = Elem<WF_F32>;
    hipLaunchKernelGGL(ee_tree_sweep_kernel<WF_F32>, dim3(blocks), dim3(kEeThreads), 0, stream, a,
                       plan.splits, plan.chunk / E::kPerVec, a.V / E::kPerVec, part);
  }
  return hipGetLastError();
}

}  // namespace wf
