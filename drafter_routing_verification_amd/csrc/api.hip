// C ABI of libwhiflash: host-side validation, workspace carving and launches.
// Every check here runs before any HIP call, so a rejected call launches
// nothing and touches no device state.
#include <stdint.h>

#include "accept.h"
#include "common.h"

namespace {

constexpr size_t kWorkspaceAlign = 256;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

inline int32_t elem_bytes(int32_t dtype) { return dtype == WF_BF16 ? 2 : 4; }

inline bool valid_dtype(int32_t dtype) { return dtype == WF_F32 || dtype == WF_BF16; }

int32_t check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return WF_OK;
  if (ws == nullptr || reinterpret_cast<uintptr_t>(ws) % kWorkspaceAlign != 0 || have < need)
    return WF_ERR_WORKSPACE;
  return WF_OK;
}

// Shared checks of the logits operand.
int32_t check_logits(const void* logits, int32_t dtype, int32_t rows, int32_t V, int64_t row_stride) {
  if (!valid_dtype(dtype)) return WF_ERR_DTYPE;
  if (V <= 0 || rows < 0 || row_stride < V) return WF_ERR_SHAPE;
  // The byte offset of every row, rows * row_stride * element size, must fit in int64.
  if (row_stride > INT64_MAX / 16 / (rows > 0 ? rows : 1)) return WF_ERR_SHAPE;
  if (rows > 0 && logits == nullptr) return WF_ERR_NULL;
  if (!aligned16(logits) || (row_stride * elem_bytes(dtype)) % 16 != 0) return WF_ERR_ALIGN;
  const wf::SweepPlan plan = wf::sweep_plan(rows, V);
  // 1-D grid of workgroups of up to 1024 threads: keep the work-item count below 2^32.
  if (static_cast<int64_t>(rows) * plan.splits * 1024 >= (int64_t{1} << 32))
    return WF_ERR_SHAPE;
  return WF_OK;
}

int32_t launch_status(hipError_t e) { return e == hipSuccess ? WF_OK : WF_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* whiflash_status_string(int32_t status) {
  switch (status) {
    case WF_OK: return "WF_OK";
    case WF_ERR_NULL: return "WF_ERR_NULL: a required pointer is NULL";
    case WF_ERR_SHAPE: return "WF_ERR_SHAPE: a size is out of range";
    case WF_ERR_DTYPE: return "WF_ERR_DTYPE: unknown element type";
    case WF_ERR_ALIGN: return "WF_ERR_ALIGN: logits base or row stride not 16-byte aligned";
    case WF_ERR_WORKSPACE: return "WF_ERR_WORKSPACE: workspace NULL, not 256-byte aligned, or too small";
    case WF_ERR_LAUNCH: return "WF_ERR_LAUNCH: kernel launch failed";
    case WF_ERR_SCRATCH:
      return "WF_ERR_SCRATCH: the round needs more than the fixed scratch of the "
             "no-allocation entry point";
    case WF_ERR_RUNTIME: return "WF_ERR_RUNTIME: a HIP runtime query failed";
    default: return "unknown whiflash status";
  }
}

size_t whiflash_route_workspace_bytes(int32_t B, int32_t m) {
  if (B <= 0 || m <= 0) return 0;
  // Pre-activation partials zp[slices][B][m] (float32), slices bounded independently of d.
  const size_t slices = static_cast<size_t>(wf::router_max_slices(B, m));
  return round_up(slices * static_cast<size_t>(B) * static_cast<size_t>(m) * sizeof(float),
                  kWorkspaceAlign);
}

size_t whiflash_verify_workspace_bytes(int32_t total_rows, int32_t V) {
  if (total_rows <= 0 || V <= 0) return 0;
  const wf::SweepPlan plan = wf::sweep_plan(total_rows, V);
  return round_up(static_cast<size_t>(total_rows) * plan.splits * sizeof(wf::Partial), kWorkspaceAlign);
}

int32_t whiflash_argmax_sweep_plan(int32_t rows, int32_t V, int32_t* chunks, int32_t* chunk_elems) {
  if (rows < 1 || V < 1) return WF_ERR_SHAPE;
  if (!chunks || !chunk_elems) return WF_ERR_NULL;
  const wf::SweepPlan plan = wf::sweep_plan(rows, V);
  *chunks = plan.splits;
  *chunk_elems = plan.chunk;
  return WF_OK;
}

int32_t whiflash_stream_read(const void* logits, int32_t dtype, int32_t rows, int32_t V,
                             int64_t row_stride, uint32_t* sink, hipStream_t stream) {
  const int32_t s = check_logits(logits, dtype, rows, V, row_stride);
  if (s != WF_OK) return s;
  if (rows == 0) return WF_OK;
  if (!sink) return WF_ERR_NULL;
  return launch_status(wf::launch_stream_read(logits, dtype, row_stride, rows, V,
                                              wf::sweep_plan(rows, V), sink, stream));
}

int32_t whiflash_argmax_sweep(const void* logits, int32_t dtype, int32_t rows, int32_t V,
                              int64_t row_stride, void* partials, size_t partials_bytes,
                              hipStream_t stream) {
  int32_t s = check_logits(logits, dtype, rows, V, row_stride);
  if (s != WF_OK) return s;
  if (rows == 0) return WF_OK;
  const wf::SweepPlan plan = wf::sweep_plan(rows, V);
  const size_t need = static_cast<size_t>(rows) * plan.splits * sizeof(wf::Partial);
  if ((s = check_workspace(partials, partials_bytes, need)) != WF_OK) return s;
  return launch_status(wf::launch_sweep(logits, dtype, row_stride, rows, V, plan,
                                        static_cast<wf::Partial*>(partials), stream));
}

}  // extern "C"

namespace {

int32_t route_impl(const void* hidden, const wf::HiddenSel& sel, int32_t dtype, int32_t B,
                   int32_t d, const void* W1, const float* b1, int32_t m, const void* W2,
                   const float* b2, float tau, float* delta_al, int32_t* choice, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return WF_ERR_DTYPE;
  if (B < 0 || d <= 0 || m <= 0) return WF_ERR_SHAPE;
  if (B == 0) return WF_OK;
  if (!hidden || !W1 || !W2 || !delta_al || !choice) return WF_ERR_NULL;
  if (static_cast<int64_t>(B) * m * wf::kMaxRouterSlices > INT32_MAX ||
      static_cast<int64_t>(m) * d > (int64_t{1} << 40) || B > 65535 ||
      d > wf::kMaxHidden)
    return WF_ERR_SHAPE;
  const int32_t s = check_workspace(workspace, workspace_bytes, whiflash_route_workspace_bytes(B, m));
  if (s != WF_OK) return s;
  float* zp = static_cast<float*>(workspace);
  const wf::RouterPlan plan = wf::router_plan(dtype, B, d, m, hidden, W1);
  if (wf::launch_router_stage1(plan, hidden, sel, dtype, B, d, W1, m, zp, stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  return launch_status(wf::launch_router_finish(plan, sel, dtype, zp, B, m, b1, W2, b2, tau,
                                                delta_al, choice, stream));
}

}  // namespace

extern "C" {

int32_t whiflash_route(const void* hidden, int32_t dtype, int32_t B, int32_t d, const void* W1,
                       const float* b1, int32_t m, const void* W2, const float* b2, float tau,
                       float* delta_al, int32_t* choice, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  const wf::HiddenSel direct{nullptr, nullptr, 0, 0};
  return route_impl(hidden, direct, dtype, B, d, W1, b1, m, W2, b2, tau, delta_al, choice,
                    workspace, workspace_bytes, stream);
}

int32_t whiflash_route_gather(const void* hidden_rows, int32_t dtype, int32_t total_rows,
                              int32_t d, int32_t B, const int32_t* row0, int32_t rows_per_seq,
                              const int32_t* pos, const void* W1, const float* b1, int32_t m,
                              const void* W2, const float* b2, float tau, float* delta_al,
                              int32_t* choice, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (total_rows < 0 || (row0 == nullptr && rows_per_seq < 0)) return WF_ERR_SHAPE;
  if (B > 0 && pos == nullptr) return WF_ERR_NULL;
  if (B > 0 && total_rows == 0 && hidden_rows == nullptr) {
    // No rows at all: every sequence gets NaN / 0 from the finish kernel, but the
    // stage-1 kernels still need a base pointer; any non-null value is never read.
    hidden_rows = W1;
  }
  const wf::HiddenSel sel{row0, pos, rows_per_seq, total_rows};
  return route_impl(hidden_rows, sel, dtype, B, d, W1, b1, m, W2, b2, tau, delta_al, choice,
                    workspace, workspace_bytes, stream);
}

int32_t whiflash_verify_chain(const void* logits, int32_t dtype, int32_t B, int32_t K, int32_t V,
                              int64_t row_stride, const int32_t* draft, int32_t* accept_len,
                              int32_t* bonus, int32_t* row_argmax, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS) return WF_ERR_SHAPE;
  const int64_t rows64 = static_cast<int64_t>(B) * (K + 1);
  if (rows64 > INT32_MAX) return WF_ERR_SHAPE;
  const int32_t rows = static_cast<int32_t>(rows64);
  int32_t s = check_logits(logits, dtype, rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!accept_len || !bonus || (K > 0 && !draft)) return WF_ERR_NULL;
  const size_t need = whiflash_verify_workspace_bytes(rows, V);
  if ((s = check_workspace(workspace, workspace_bytes, need)) != WF_OK) return s;
  const wf::SweepPlan plan = wf::few_rows_plan(rows, V, K + 1);
  wf::Partial* part = static_cast<wf::Partial*>(workspace);
  if (wf::launch_sweep(logits, dtype, row_stride, rows, V, plan, part, stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  return launch_status(wf::launch_finalize_chain(part, plan.splits, B, K, draft, accept_len, bonus,
                                                 row_argmax, stream));
}

size_t whiflash_early_exit_workspace_bytes(int32_t B, int32_t K, int32_t V) {
  if (B <= 0 || K < 0 || V <= 0) return 0;
  const int64_t rows = static_cast<int64_t>(B) * (static_cast<int64_t>(K) + 1);
  if (rows > INT32_MAX) return 0;  // more rows than the call accepts
  const wf::SweepPlan plan = wf::early_exit_plan(B, V);
  // Per-sequence mismatch flags, then the chunk partials of every row.
  return round_up(static_cast<size_t>(B) * sizeof(int32_t), kWorkspaceAlign) +
         round_up(static_cast<size_t>(rows) * plan.splits * sizeof(wf::Partial), kWorkspaceAlign);
}

int32_t whiflash_verify_chain_early_exit(const void* logits, int32_t dtype, int32_t B, int32_t K,
                                         int32_t V, int64_t row_stride, const int32_t* draft,
                                         int32_t* accept_len, int32_t* bonus, int32_t* row_argmax,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  if (B < 0 || K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS) return WF_ERR_SHAPE;
  const int64_t rows64 = static_cast<int64_t>(B) * (K + 1);
  if (rows64 > INT32_MAX) return WF_ERR_SHAPE;
  const int32_t rows = static_cast<int32_t>(rows64);
  int32_t s = check_logits(logits, dtype, rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!accept_len || !bonus || (K > 0 && !draft)) return WF_ERR_NULL;
  const wf::SweepPlan plan = wf::early_exit_plan(B, V);
  if (rows64 * plan.splits * 1024 >= (int64_t{1} << 32)) return WF_ERR_SHAPE;
  const size_t need = whiflash_early_exit_workspace_bytes(B, K, V);
  if ((s = check_workspace(workspace, workspace_bytes, need)) != WF_OK) return s;
  int* flags = static_cast<int*>(workspace);
  wf::Partial* part = reinterpret_cast<wf::Partial*>(
      static_cast<char*>(workspace) + round_up(static_cast<size_t>(B) * sizeof(int32_t), kWorkspaceAlign));
  return launch_status(wf::launch_early_exit_chain(logits, dtype, row_stride, B, K, V, plan, draft,
                                                   flags, part, accept_len, bonus, row_argmax,
                                                   stream));
}

int32_t whiflash_verify_tree(const void* logits, int32_t dtype, int32_t B, int32_t N, int32_t V,
                             int64_t row_stride, const int32_t* parent, const int32_t* draft_ids,
                             const int32_t* d2t, int32_t Vd, int32_t* accept_len, int32_t* bonus,
                             int32_t* best_node, int32_t* row_argmax, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || N < 1 || N > WHIFLASH_MAX_SEQ_ROWS || Vd < 1) return WF_ERR_SHAPE;
  const int64_t rows64 = static_cast<int64_t>(B) * N;
  if (rows64 > INT32_MAX) return WF_ERR_SHAPE;
  const int32_t rows = static_cast<int32_t>(rows64);
  int32_t s = check_logits(logits, dtype, rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!parent || !draft_ids || !d2t || !accept_len || !bonus) return WF_ERR_NULL;
  const size_t need = whiflash_verify_workspace_bytes(rows, V);
  if ((s = check_workspace(workspace, workspace_bytes, need)) != WF_OK) return s;
  const wf::SweepPlan plan = wf::few_rows_plan(rows, V, N);
  wf::Partial* part = static_cast<wf::Partial*>(workspace);
  if (wf::launch_sweep(logits, dtype, row_stride, rows, V, plan, part, stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  return launch_status(wf::launch_finalize_tree(part, plan.splits, B, N, V, parent, draft_ids, d2t,
                                                Vd, accept_len, bonus, best_node, row_argmax,
                                                stream));
}

int32_t whiflash_verify_routed(const void* logits, int32_t dtype, int32_t B, int32_t V,
                               int64_t row_stride, const int32_t* row_offsets, int32_t total_rows,
                               const int32_t* choice, int32_t K, const int32_t* chain_draft,
                               int32_t N, const int32_t* parent, const int32_t* draft_ids,
                               const int32_t* d2t, int32_t Vd, int32_t* accept_len, int32_t* bonus,
                               int32_t* best_node, int32_t* row_argmax, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || total_rows < 0 || K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS || N < 1 ||
      N > WHIFLASH_MAX_SEQ_ROWS || Vd < 1)
    return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, dtype, total_rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!row_offsets || !choice || (K > 0 && !chain_draft) || !parent || !draft_ids || !d2t ||
      !accept_len || !bonus)
    return WF_ERR_NULL;
  const size_t need = whiflash_verify_workspace_bytes(total_rows, V);
  if ((s = check_workspace(workspace, workspace_bytes, need)) != WF_OK) return s;
  const wf::SweepPlan plan = wf::few_rows_plan(total_rows, V, K + 1 > N ? K + 1 : N);
  wf::Partial* part = static_cast<wf::Partial*>(workspace);
  if (wf::launch_sweep(logits, dtype, row_stride, total_rows, V, plan, part, stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  return launch_status(wf::launch_finalize_routed(false, part, plan.splits, B, V, row_offsets, total_rows,
                                                  choice, K, chain_draft, N, parent, draft_ids, d2t,
                                                  Vd, accept_len, bonus, best_node, row_argmax,
                                                  stream));
}

size_t whiflash_tree_early_exit_workspace_bytes(int32_t B, int32_t N, int32_t V) {
  if (B <= 0 || N <= 0 || N > WHIFLASH_MAX_SEQ_ROWS || V <= 0) return 0;
  const int64_t rows = static_cast<int64_t>(B) * N;
  if (rows > INT32_MAX) return 0;  // more rows than the call accepts
  return wf::ee_tree_workspace(B, N, static_cast<int32_t>(rows), V, kWorkspaceAlign).total;
}

size_t whiflash_routed_early_exit_workspace_bytes(int32_t B, int32_t K, int32_t N, int32_t total_rows,
                                                  int32_t V) {
  if (B <= 0 || K < 0 || N <= 0 || total_rows < 0 || V <= 0) return 0;
  if (K >= WHIFLASH_MAX_SEQ_ROWS) return 0;
  const int32_t rmax = K + 1 > N ? K + 1 : N;
  if (rmax > WHIFLASH_MAX_SEQ_ROWS) return 0;
  return wf::ee_tree_workspace(B, rmax, total_rows, V, kWorkspaceAlign).total;
}

size_t whiflash_round_workspace_bytes(int32_t B, int32_t m, int32_t total_rows, int32_t V) {
  if (B <= 0 || m <= 0 || V <= 0) return 0;
  return whiflash_route_workspace_bytes(B, m) + whiflash_verify_workspace_bytes(total_rows, V);
}

int32_t whiflash_round_routed(const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1,
                              const float* b1, int32_t m, const void* W2, const float* b2,
                              float tau, float* delta_al, int32_t* choice, const void* logits,
                              int32_t logits_dtype, int32_t B, int32_t V, int64_t row_stride,
                              const int32_t* row_offsets, int32_t total_rows, int32_t K,
                              const int32_t* chain_draft, int32_t N, const int32_t* parent,
                              const int32_t* draft_ids, const int32_t* d2t, int32_t Vd,
                              int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                              int32_t* row_argmax, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  // Router arguments, as whiflash_route.
  if (!valid_dtype(hidden_dtype)) return WF_ERR_DTYPE;
  if (B < 0 || d <= 0 || m <= 0) return WF_ERR_SHAPE;
  // Verify arguments, as whiflash_verify_routed.
  if (total_rows < 0 || K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS || N < 1 ||
      N > WHIFLASH_MAX_SEQ_ROWS || Vd < 1)
    return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, logits_dtype, total_rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!hidden || !W1 || !W2 || !delta_al || !choice) return WF_ERR_NULL;
  if (!row_offsets || (K > 0 && !chain_draft) || !parent || !draft_ids || !d2t || !accept_len ||
      !bonus)
    return WF_ERR_NULL;
  if (static_cast<int64_t>(B) * m * wf::kMaxRouterSlices > INT32_MAX ||
      static_cast<int64_t>(m) * d > (int64_t{1} << 40) || B > 65535 ||
      d > wf::kMaxHidden)
    return WF_ERR_SHAPE;
  const size_t route_bytes = whiflash_route_workspace_bytes(B, m);
  if ((s = check_workspace(workspace, workspace_bytes,
                           whiflash_round_workspace_bytes(B, m, total_rows, V))) != WF_OK)
    return s;
  float* zp = static_cast<float*>(workspace);
  wf::Partial* part = reinterpret_cast<wf::Partial*>(static_cast<char*>(workspace) + route_bytes);
  const wf::RouterPlan plan = wf::router_plan(hidden_dtype, B, d, m, hidden, W1);
  const bool fused = wf::round_stage1_fused(plan, hidden_dtype, hidden, B, d, W1);
  const wf::SweepPlan sp = fused ? wf::few_rows_plan(total_rows, V, K + 1 > N ? K + 1 : N)
                                 : wf::sweep_plan(total_rows, V);
  const wf::RoutedArgs args{part, sp.splits, V, row_offsets, total_rows, K, chain_draft, N, parent,
                            draft_ids, d2t, Vd, accept_len, bonus, best_node, row_argmax};
  if (wf::launch_round_stage1(fused, plan, hidden_dtype, hidden, B, d, W1, m, zp, logits,
                              logits_dtype, row_stride, total_rows, V, sp, part,
                              stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  return launch_status(wf::launch_round_finalize(hidden_dtype, plan, zp, B, m, b1, W2, b2, tau,
                                                 delta_al, choice, args, stream));
}

int32_t whiflash_catchup_update(int32_t B, const int32_t* cur_choice, const int32_t* accept_len,
                                const int32_t* next_choice, int32_t* backlog, int32_t* switch_flag,
                                int32_t* catchup_len, hipStream_t stream) {
  if (B < 0) return WF_ERR_SHAPE;
  if (B == 0) return WF_OK;
  if (!cur_choice || !accept_len || !next_choice || !backlog) return WF_ERR_NULL;
  return launch_status(wf::launch_catchup(B, cur_choice, accept_len, next_choice, backlog,
                                          switch_flag, catchup_len, stream));
}

size_t whiflash_entropy_workspace_bytes(int32_t B, int32_t V) {
  if (B <= 0 || V <= 0) return 0;
  const wf::SweepPlan plan = wf::entropy_plan(B, V);
  return round_up(static_cast<size_t>(B) * plan.splits * 16, kWorkspaceAlign);
}

int32_t whiflash_route_entropy(const void* logits, int32_t dtype, int32_t total_rows, int32_t V,
                               int64_t row_stride, int32_t B, const int32_t* row0,
                               int32_t rows_per_seq, const int32_t* pos, float tau,
                               float* entropy, int32_t* choice, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || total_rows < 0 || (row0 == nullptr && rows_per_seq < 0)) return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, dtype, total_rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (B > INT32_MAX / 64) return WF_ERR_SHAPE;
  if (!pos || !entropy || !choice) return WF_ERR_NULL;
  if ((s = check_workspace(workspace, workspace_bytes, whiflash_entropy_workspace_bytes(B, V))) != WF_OK)
    return s;
  return launch_status(wf::launch_entropy(logits, dtype, row_stride, total_rows, V, B, row0,
                                          rows_per_seq, pos, tau, entropy, choice, workspace,
                                          stream));
}

size_t whiflash_round_early_exit_workspace_bytes(int32_t B, int32_t m, int32_t K, int32_t N,
                                                 int32_t total_rows, int32_t V) {
  if (B <= 0 || m <= 0 || V <= 0) return 0;
  const size_t ee = whiflash_routed_early_exit_workspace_bytes(B, K, N, total_rows, V);
  return ee == 0 ? 0 : whiflash_route_workspace_bytes(B, m) + ee;
}

}  // extern "C"

namespace {

// Shared body of the early-exit tree / routed entry points: prep (or the
// round's router finish + prep), node-major sweep, masked routed acceptance.
// `zp` non-NULL means a fused round whose router stage 1 is already launched.
int32_t ee_tree_impl(const void* logits, int32_t dtype, int32_t B, int32_t V, int64_t row_stride,
                     const int32_t* row_offsets, int32_t total_rows, const int32_t* choice,
                     int32_t K, const int32_t* chain_draft, int32_t N, const int32_t* parent,
                     const int32_t* draft_ids, const int32_t* d2t, int32_t Vd, int32_t* accept_len,
                     int32_t* bonus, int32_t* best_node, int32_t* row_argmax, char* ws,
                     hipStream_t stream, const wf::RouterPlan* rplan, int32_t hidden_dtype,
                     const float* zp, int32_t m, const float* b1, const void* W2, const float* b2,
                     float tau, float* delta_al, int32_t* route_choice) {
  const int32_t rmax = row_offsets ? (K + 1 > N ? K + 1 : N) : N;
  const wf::EeTreeWs off = wf::ee_tree_workspace(B, rmax, total_rows, V, kWorkspaceAlign);
  const wf::SweepPlan plan = wf::early_exit_plan(B, V);
  const wf::EeTreeArgs a = wf::ee_tree_args(ws, off, B, rmax, logits, dtype, row_stride, V,
                                            row_offsets, row_offsets ? choice : nullptr,
                                            total_rows, K, chain_draft, N, parent, draft_ids, d2t,
                                            Vd);
  wf::Partial* part = reinterpret_cast<wf::Partial*>(ws + off.part);
  hipError_t e = rplan ? wf::launch_ee_round_prep(a, hidden_dtype, *rplan, zp, m, b1, W2, b2, tau,
                                                  delta_al, route_choice, stream)
                       : wf::launch_ee_tree_prep(a, stream);
  if (e != hipSuccess) return WF_ERR_LAUNCH;
  if (wf::launch_ee_tree_sweep(a, plan, part, stream) != hipSuccess) return WF_ERR_LAUNCH;
  const int32_t* offs = row_offsets ? row_offsets : a.seq_off;
  const int32_t* ch = row_offsets ? choice : a.seq_choice;
  const int32_t rows_total = row_offsets ? total_rows : B * N;
  return launch_status(wf::launch_finalize_routed(true, part, plan.splits, B, V, offs, rows_total, ch,
                                                  row_offsets ? K : 0, chain_draft, N, parent,
                                                  draft_ids, d2t, Vd, accept_len, bonus, best_node,
                                                  row_argmax, stream));
}

// Grid of the node-major sweep: rmax * B * splits workgroups of up to 1024 threads.
bool ee_grid_ok(int32_t B, int32_t rmax, int32_t V) {
  const wf::SweepPlan plan = wf::early_exit_plan(B, V);
  return static_cast<int64_t>(rmax) * B * plan.splits * 1024 < (int64_t{1} << 32);
}

}  // namespace

extern "C" {

int32_t whiflash_verify_tree_early_exit(const void* logits, int32_t dtype, int32_t B, int32_t N,
                                        int32_t V, int64_t row_stride, const int32_t* parent,
                                        const int32_t* draft_ids, const int32_t* d2t, int32_t Vd,
                                        int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                                        int32_t* row_argmax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || N < 1 || N > WHIFLASH_MAX_SEQ_ROWS || Vd < 1) return WF_ERR_SHAPE;
  const int64_t rows64 = static_cast<int64_t>(B) * N;
  if (rows64 > INT32_MAX) return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, dtype, static_cast<int32_t>(rows64), V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!parent || !draft_ids || !d2t || !accept_len || !bonus) return WF_ERR_NULL;
  if (!ee_grid_ok(B, N, V)) return WF_ERR_SHAPE;
  if ((s = check_workspace(workspace, workspace_bytes,
                           whiflash_tree_early_exit_workspace_bytes(B, N, V))) != WF_OK)
    return s;
  return ee_tree_impl(logits, dtype, B, V, row_stride, nullptr, static_cast<int32_t>(rows64),
                      nullptr, 0, nullptr, N, parent, draft_ids, d2t, Vd, accept_len, bonus,
                      best_node, row_argmax, static_cast<char*>(workspace), stream, nullptr, 0,
                      nullptr, 0, nullptr, nullptr, nullptr, 0.0f, nullptr, nullptr);
}

int32_t whiflash_verify_routed_early_exit(const void* logits, int32_t dtype, int32_t B, int32_t V,
                                          int64_t row_stride, const int32_t* row_offsets,
                                          int32_t total_rows, const int32_t* choice, int32_t K,
                                          const int32_t* chain_draft, int32_t N,
                                          const int32_t* parent, const int32_t* draft_ids,
                                          const int32_t* d2t, int32_t Vd, int32_t* accept_len,
                                          int32_t* bonus, int32_t* best_node, int32_t* row_argmax,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  if (B < 0 || total_rows < 0 || K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS || N < 1 ||
      N > WHIFLASH_MAX_SEQ_ROWS || Vd < 1)
    return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, dtype, total_rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!row_offsets || !choice || (K > 0 && !chain_draft) || !parent || !draft_ids || !d2t ||
      !accept_len || !bonus)
    return WF_ERR_NULL;
  if (!ee_grid_ok(B, K + 1 > N ? K + 1 : N, V)) return WF_ERR_SHAPE;
  if ((s = check_workspace(workspace, workspace_bytes,
                           whiflash_routed_early_exit_workspace_bytes(B, K, N, total_rows, V))) !=
      WF_OK)
    return s;
  return ee_tree_impl(logits, dtype, B, V, row_stride, row_offsets, total_rows, choice, K,
                      chain_draft, N, parent, draft_ids, d2t, Vd, accept_len, bonus, best_node,
                      row_argmax, static_cast<char*>(workspace), stream, nullptr, 0, nullptr, 0,
                      nullptr, nullptr, nullptr, 0.0f, nullptr, nullptr);
}

int32_t whiflash_round_routed_early_exit(
    const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1, const float* b1, int32_t m,
    const void* W2, const float* b2, float tau, float* delta_al, int32_t* choice,
    const void* logits, int32_t logits_dtype, int32_t B, int32_t V, int64_t row_stride,
    const int32_t* row_offsets, int32_t total_rows, int32_t K, const int32_t* chain_draft,
    int32_t N, const int32_t* parent, const int32_t* draft_ids, const int32_t* d2t, int32_t Vd,
    int32_t* accept_len, int32_t* bonus, int32_t* best_node, int32_t* row_argmax, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(hidden_dtype)) return WF_ERR_DTYPE;
  if (B < 0 || d <= 0 || m <= 0) return WF_ERR_SHAPE;
  if (total_rows < 0 || K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS || N < 1 ||
      N > WHIFLASH_MAX_SEQ_ROWS || Vd < 1)
    return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, logits_dtype, total_rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!hidden || !W1 || !W2 || !delta_al || !choice) return WF_ERR_NULL;
  if (!row_offsets || (K > 0 && !chain_draft) || !parent || !draft_ids || !d2t || !accept_len ||
      !bonus)
    return WF_ERR_NULL;
  if (static_cast<int64_t>(B) * m * wf::kMaxRouterSlices > INT32_MAX ||
      static_cast<int64_t>(m) * d > (int64_t{1} << 40) || B > 65535 ||
      d > wf::kMaxHidden)
    return WF_ERR_SHAPE;
  if (!ee_grid_ok(B, K + 1 > N ? K + 1 : N, V)) return WF_ERR_SHAPE;
  if ((s = check_workspace(workspace, workspace_bytes,
                           whiflash_round_early_exit_workspace_bytes(B, m, K, N, total_rows, V))) !=
      WF_OK)
    return s;
  const size_t route_bytes = whiflash_route_workspace_bytes(B, m);
  float* zp = static_cast<float*>(workspace);
  const wf::HiddenSel direct{nullptr, nullptr, 0, 0};
  const wf::RouterPlan plan = wf::router_plan(hidden_dtype, B, d, m, hidden, W1);
  if (wf::launch_router_stage1(plan, hidden, direct, hidden_dtype, B, d, W1, m, zp, stream) !=
      hipSuccess)
    return WF_ERR_LAUNCH;
  return ee_tree_impl(logits, logits_dtype, B, V, row_stride, row_offsets, total_rows, choice, K,
                      chain_draft, N, parent, draft_ids, d2t, Vd, accept_len, bonus, best_node,
                      row_argmax, static_cast<char*>(workspace) + route_bytes, stream, &plan,
                      hidden_dtype, zp, m, b1, W2, b2, tau, delta_al, choice);
}

size_t whiflash_verify_routed_entropy_workspace_bytes(int32_t B, int32_t total_rows, int32_t V) {
  if (B <= 0 || total_rows <= 0 || V <= 0) return 0;
  // Chunk partials of the sweep, the best nodes when the caller passes none,
  // then the entropy pass's partials.
  return whiflash_verify_workspace_bytes(total_rows, V) +
         round_up(static_cast<size_t>(B) * sizeof(int32_t), kWorkspaceAlign) +
         whiflash_entropy_workspace_bytes(B, V);
}

int32_t whiflash_verify_routed_entropy(const void* logits, int32_t dtype, int32_t B, int32_t V,
                                       int64_t row_stride, const int32_t* row_offsets,
                                       int32_t total_rows, const int32_t* choice, int32_t K,
                                       const int32_t* chain_draft, int32_t N,
                                       const int32_t* parent, const int32_t* draft_ids,
                                       const int32_t* d2t, int32_t Vd, float tau_entropy,
                                       int32_t* accept_len, int32_t* bonus, int32_t* best_node,
                                       int32_t* row_argmax, float* entropy, int32_t* next_choice,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if (B < 0 || total_rows < 0 || K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS || N < 1 ||
      N > WHIFLASH_MAX_SEQ_ROWS || Vd < 1)
    return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, dtype, total_rows, V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (B > INT32_MAX / 64) return WF_ERR_SHAPE;
  if (!row_offsets || !choice || (K > 0 && !chain_draft) || !parent || !draft_ids || !d2t ||
      !accept_len || !bonus || !entropy || !next_choice)
    return WF_ERR_NULL;
  if ((s = check_workspace(workspace, workspace_bytes,
                           whiflash_verify_routed_entropy_workspace_bytes(B, total_rows, V))) !=
      WF_OK)
    return s;
  char* ws = static_cast<char*>(workspace);
  const size_t part_bytes = whiflash_verify_workspace_bytes(total_rows, V);
  const size_t best_bytes = round_up(static_cast<size_t>(B) * sizeof(int32_t), kWorkspaceAlign);
  const wf::SweepPlan plan = wf::few_rows_plan(total_rows, V, K + 1 > N ? K + 1 : N);
  wf::Partial* part = reinterpret_cast<wf::Partial*>(ws);
  int32_t* best = best_node ? best_node : reinterpret_cast<int32_t*>(ws + part_bytes);
  if (wf::launch_sweep(logits, dtype, row_stride, total_rows, V, plan, part, stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  if (wf::launch_finalize_routed(false, part, plan.splits, B, V, row_offsets, total_rows, choice, K,
                                 chain_draft, N, parent, draft_ids, d2t, Vd, accept_len, bonus,
                                 best, row_argmax, stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  // Malformed sequences have best node -1, which selects no row: H = NaN, choice 0.
  return launch_status(wf::launch_entropy(logits, dtype, row_stride, total_rows, V, B, row_offsets,
                                          0, best, tau_entropy, entropy, next_choice,
                                          ws + part_bytes + best_bytes, stream));
}

size_t whiflash_round_chain_workspace_bytes(int32_t B, int32_t m, int32_t K, int32_t V) {
  if (B <= 0 || m <= 0 || K < 0 || V <= 0) return 0;
  const int64_t rows = static_cast<int64_t>(B) * (static_cast<int64_t>(K) + 1);
  if (rows > INT32_MAX) return 0;  // more rows than the call accepts
  return whiflash_route_workspace_bytes(B, m) +
         whiflash_verify_workspace_bytes(static_cast<int32_t>(rows), V);
}

}  // extern "C"

namespace wf {

// Every check of whiflash_round_chain's arguments except the workspace's.
int32_t round_chain_check(const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1,
                          int32_t m, const void* W2, const float* delta_al, const int32_t* choice,
                          const void* logits, int32_t logits_dtype, int32_t B, int32_t K, int32_t V,
                          int64_t row_stride, const int32_t* draft, const int32_t* accept_len,
                          const int32_t* bonus) {
  // Router arguments, as whiflash_route.
  if (!valid_dtype(hidden_dtype)) return WF_ERR_DTYPE;
  if (B < 0 || d <= 0 || m <= 0) return WF_ERR_SHAPE;
  // Verify arguments, as whiflash_verify_chain.
  if (K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS) return WF_ERR_SHAPE;
  const int64_t rows64 = static_cast<int64_t>(B) * (K + 1);
  if (rows64 > INT32_MAX) return WF_ERR_SHAPE;
  const int32_t s = check_logits(logits, logits_dtype, static_cast<int32_t>(rows64), V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!hidden || !W1 || !W2 || !delta_al || !choice) return WF_ERR_NULL;
  if (!accept_len || !bonus || (K > 0 && !draft)) return WF_ERR_NULL;
  if (static_cast<int64_t>(B) * m * kMaxRouterSlices > INT32_MAX ||
      static_cast<int64_t>(m) * d > (int64_t{1} << 40) || B > 65535 ||
      d > wf::kMaxHidden)
    return WF_ERR_SHAPE;
  return WF_OK;
}

}  // namespace wf

extern "C" {

int32_t whiflash_round_chain(const void* hidden, int32_t hidden_dtype, int32_t d, const void* W1,
                             const float* b1, int32_t m, const void* W2, const float* b2,
                             float tau, float* delta_al, int32_t* choice, const void* logits,
                             int32_t logits_dtype, int32_t B, int32_t K, int32_t V,
                             int64_t row_stride, const int32_t* draft, int32_t* accept_len,
                             int32_t* bonus, int32_t* row_argmax, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  int32_t s = wf::round_chain_check(hidden, hidden_dtype, d, W1, m, W2, delta_al, choice, logits,
                                    logits_dtype, B, K, V, row_stride, draft, accept_len, bonus);
  if (s != WF_OK || B == 0) return s;
  const int32_t rows = B * (K + 1);
  if ((s = check_workspace(workspace, workspace_bytes,
                           whiflash_round_chain_workspace_bytes(B, m, K, V))) != WF_OK)
    return s;
  const size_t route_bytes = whiflash_route_workspace_bytes(B, m);
  float* zp = static_cast<float*>(workspace);
  wf::Partial* part = reinterpret_cast<wf::Partial*>(static_cast<char*>(workspace) + route_bytes);
  const wf::RouterPlan plan = wf::router_plan(hidden_dtype, B, d, m, hidden, W1);
  const bool fused = wf::round_stage1_fused(plan, hidden_dtype, hidden, B, d, W1);
  const wf::SweepPlan sp = fused ? wf::few_rows_plan(rows, V, K + 1) : wf::sweep_plan(rows, V);
  if (wf::launch_round_stage1(fused, plan, hidden_dtype, hidden, B, d, W1, m, zp, logits,
                              logits_dtype, row_stride, rows, V, sp, part, stream) != hipSuccess)
    return WF_ERR_LAUNCH;
  return launch_status(wf::launch_round_chain_finalize(hidden_dtype, plan, zp, B, m, b1, W2, b2,
                                                       tau, delta_al, choice, part, sp.splits, K,
                                                       draft, accept_len, bonus, row_argmax,
                                                       stream));
}

size_t whiflash_round_chain_early_exit_workspace_bytes(int32_t B, int32_t m, int32_t K,
                                                       int32_t V) {
  if (B <= 0 || m <= 0 || K < 0 || V <= 0) return 0;
  const size_t ee = whiflash_early_exit_workspace_bytes(B, K, V);
  return ee == 0 ? 0 : whiflash_route_workspace_bytes(B, m) + ee;
}

int32_t whiflash_round_chain_early_exit(const void* hidden, int32_t hidden_dtype, int32_t d,
                                        const void* W1, const float* b1, int32_t m, const void* W2,
                                        const float* b2, float tau, float* delta_al,
                                        int32_t* choice, const void* logits, int32_t logits_dtype,
                                        int32_t B, int32_t K, int32_t V, int64_t row_stride,
                                        const int32_t* draft, int32_t* accept_len, int32_t* bonus,
                                        int32_t* row_argmax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(hidden_dtype)) return WF_ERR_DTYPE;
  if (B < 0 || d <= 0 || m <= 0) return WF_ERR_SHAPE;
  if (K < 0 || K >= WHIFLASH_MAX_SEQ_ROWS) return WF_ERR_SHAPE;
  const int64_t rows64 = static_cast<int64_t>(B) * (K + 1);
  if (rows64 > INT32_MAX) return WF_ERR_SHAPE;
  int32_t s = check_logits(logits, logits_dtype, static_cast<int32_t>(rows64), V, row_stride);
  if (s != WF_OK) return s;
  if (B == 0) return WF_OK;
  if (!hidden || !W1 || !W2 || !delta_al || !choice) return WF_ERR_NULL;
  if (!accept_len || !bonus || (K > 0 && !draft)) return WF_ERR_NULL;
  if (static_cast<int64_t>(B) * m * wf::kMaxRouterSlices > INT32_MAX ||
      static_cast<int64_t>(m) * d > (int64_t{1} << 40) || B > 65535 ||
      d > wf::kMaxHidden)
    return WF_ERR_SHAPE;
  const wf::SweepPlan plan = wf::early_exit_plan(B, V);
  if (rows64 * plan.splits * 1024 >= (int64_t{1} << 32)) return WF_ERR_SHAPE;
  if ((s = check_workspace(workspace, workspace_bytes,
                           whiflash_round_chain_early_exit_workspace_bytes(B, m, K, V))) != WF_OK)
    return s;
  char* ws = static_cast<char*>(workspace);
  const size_t route_bytes = whiflash_route_workspace_bytes(B, m);
  float* zp = reinterpret_cast<float*>(ws);
  int* flags = reinterpret_cast<int*>(ws + route_bytes);
  wf::Partial* part = reinterpret_cast<wf::Partial*>(
      ws + route_bytes + round_up(static_cast<size_t>(B) * sizeof(int32_t), kWorkspaceAlign));
  const wf::HiddenSel direct{nullptr, nullptr, 0, 0};
  const wf::RouterPlan rplan = wf::router_plan(hidden_dtype, B, d, m, hidden, W1);
  // Router stage 1 also clears the per-sequence mismatch flags.
  if (wf::launch_router_stage1(rplan, hidden, direct, hidden_dtype, B, d, W1, m, zp, stream,
                               wf::ZeroFill{flags, B}) != hipSuccess)
    return WF_ERR_LAUNCH;
  return launch_status(wf::launch_early_exit_round(logits, logits_dtype, row_stride, B, K, V, plan,
                                                   draft, flags, part, hidden_dtype, rplan, zp, m,
                                                   b1, W2, b2, tau, delta_al, choice, accept_len,
                                                   bonus, row_argmax, stream));
}

}  // extern "C"
