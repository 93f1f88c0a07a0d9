// whiflash_round_chain for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// round's scratch (router partial sums and the sweep's per-chunk records) lives
// in one fixed array of device memory that the library's code object holds, so
// the caller passes inputs and outputs only.
//
// The array `scratch` is a device symbol.  In host code its name is a host-side
// stand-in, not a device address, so the host never passes it to a kernel: on
// the first call on each device it asks the runtime for that device's address of
// the array (hipGetSymbolAddress, with that device current) and keeps it.  Every
// later call on the device uses the kept address.
#include <atomic>
#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = WHIFLASH_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on `dev`, looked up once per device.
int32_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return WF_ERR_RUNTIME;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) {
    *out = p;
    return WF_OK;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return WF_ERR_RUNTIME;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return WF_ERR_RUNTIME;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return WF_ERR_RUNTIME;
    if (e != hipSuccess || p == nullptr) return WF_ERR_RUNTIME;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return WF_OK;
}

}  // namespace

extern "C" {

int32_t whiflash_round_chain_noalloc(const void* hidden, int32_t hidden_dtype, int32_t d,
                                     const void* W1, const float* b1, int32_t m, const void* W2,
                                     const float* b2, float tau, float* delta_al, int32_t* choice,
                                     const void* logits, int32_t logits_dtype, int32_t B,
                                     int32_t K, int32_t V, int64_t row_stride,
                                     const int32_t* draft, int32_t* accept_len, int32_t* bonus,
                                     int32_t* row_argmax, hipStream_t stream) {
  // The arguments are checked as whiflash_round_chain checks them, before any HIP call.
  const int32_t c = wf::round_chain_check(hidden, hidden_dtype, d, W1, m, W2, delta_al, choice,
                                          logits, logits_dtype, B, K, V, row_stride, draft,
                                          accept_len, bonus);
  if (c != WF_OK || B == 0) return c;
  if (whiflash_round_chain_workspace_bytes(B, m, K, V) > kScratchBytes) return WF_ERR_SCRATCH;
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return WF_ERR_RUNTIME;
  void* ws = nullptr;
  const int32_t s = scratch_address(dev, &ws);
  if (s != WF_OK) return s;
  // Every byte of the scratch that the round reads it first writes (router partial
  // sums, then per-chunk records), so nothing needs clearing between calls.
  return whiflash_round_chain(hidden, hidden_dtype, d, W1, b1, m, W2, b2, tau, delta_al, choice,
                              logits, logits_dtype, B, K, V, row_stride, draft, accept_len, bonus,
                              row_argmax, ws, kScratchBytes, stream);
}

}  // extern "C"
