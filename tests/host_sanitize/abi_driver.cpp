// Host-side run of libwhiflash's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU.  The library's sources are compiled
// for the host only; this file stands in for the HIP runtime entry points they
// call (kernel registration, launch configuration, hipLaunchKernel, device
// queries).  The launch stand-in runs nothing: it records each kernel's name
// and grid, so the driver can check every launch shape against the sizes the
// call was given.  Exit status 0 means every check passed (the sanitizers abort
// on the first error they find).
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <string>
#include <vector>

#include "interleave.h"
#include "whiflash.h"

// ----------------------------------------------------------------------------- HIP stand-ins

namespace {

struct Launch {
  std::string name;
  dim3 grid, block;
};

std::map<const void*, std::string> g_names;
std::vector<Launch> g_launches;
dim3 g_grid, g_block;
int g_failures = 0;

void fail(const char* what, const char* detail) {
  fprintf(stderr, "FAIL: %s (%s)\n", what, detail);
  ++g_failures;
}

}  // namespace

extern "C" {

void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void* host_fn, char*, const char* device_name,
                           unsigned int, uint3*, uint3*, dim3*, dim3*, int*) {
  g_names[host_fn] = device_name;
}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t, hipStream_t) {
  g_grid = grid;
  g_block = block;
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  *grid = g_grid;
  *block = g_block;
  *shmem = 0;
  *stream = nullptr;
  return hipSuccess;
}
hipError_t hipLaunchKernel(const void* fn, dim3 grid, dim3 block, void**, size_t, hipStream_t) {
  auto it = g_names.find(fn);
  g_launches.push_back(Launch{it == g_names.end() ? std::string("?") : it->second, grid, block});
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void*) {
  *p = reinterpret_cast<void*>(uintptr_t{1} << 40);  // a fake, 256-byte aligned device address
  return hipSuccess;
}

}  // extern "C"

// ----------------------------------------------------------------------------- checks

namespace {

const void* const A = reinterpret_cast<const void*>(uintptr_t{1} << 20);  // fake device data
void* const W = reinterpret_cast<void*>(uintptr_t{1} << 32);              // fake workspace
const size_t kBig = size_t{1} << 40;
const int32_t V = 151936;

#define EXPECT(cond, detail)            \
  do {                                  \
    if (!(cond)) fail(#cond, (detail)); \
  } while (0)

bool has(const char* kernel) {
  for (const Launch& l : g_launches)
    if (l.name.find(kernel) != std::string::npos) return true;
  return false;
}

// Every recorded launch: a non-empty grid within the hardware limits and a 64-multiple
// block of at most 1024 threads, with fewer than 2^32 work-items along x.
void check_shapes(const char* call) {
  EXPECT(!g_launches.empty(), call);
  for (const Launch& l : g_launches) {
    const uint64_t items = uint64_t{l.grid.x} * l.block.x;
    EXPECT(l.grid.x >= 1 && l.grid.y >= 1 && l.grid.z >= 1, l.name.c_str());
    EXPECT(l.grid.y <= 65535 && l.grid.z <= 65535, l.name.c_str());
    EXPECT(l.block.x >= 64 && l.block.x <= 1024 && l.block.x % 64 == 0, l.name.c_str());
    EXPECT(l.block.y == 1 && l.block.z == 1, l.name.c_str());
    EXPECT(items < (uint64_t{1} << 32), l.name.c_str());
  }
}

// The argmax sweep launch of `rows` rows covers rows * c workgroups: c = the public plan's
// chunk count when `exact`, else (the verify calls' one-pass cap at small batches) a whole
// number of chunks per row no larger than it.
void check_sweep(const char* call, int32_t rows, int32_t v, bool exact = false) {
  int32_t chunks = 0, elems = 0;
  EXPECT(whiflash_argmax_sweep_plan(rows, v, &chunks, &elems) == WF_OK, call);
  bool seen = false;
  for (const Launch& l : g_launches)
    if (l.name.find("argmax_sweep_kernel") != std::string::npos) {
      seen = true;
      const uint64_t g = l.grid.x;
      if (exact) {
        EXPECT(g == uint64_t(rows) * chunks, call);
      } else {
        EXPECT(g % rows == 0 && g / rows >= 1 && g / rows <= uint64_t(chunks), call);
      }
    }
  EXPECT(seen, call);
}

void check_per_sequence(const char* call, const char* kernel, int32_t B) {
  bool seen = false;
  for (const Launch& l : g_launches)
    if (l.name.find(kernel) != std::string::npos) {
      seen = true;
      EXPECT(int64_t(l.grid.x) * l.grid.y * l.grid.z == B, call);
    }
  EXPECT(seen, call);
}

void plans() {
  const int32_t vs[] = {1, 7, 255, 256, 257, 2048, 3001, 20011, 128256, 151936, 262144, 1000003,
                        INT32_MAX / 2};
  const int32_t rs[] = {1, 2, 17, 61, 136, 544, 4352, 4992, 65536, 1 << 22, INT32_MAX};
  for (int32_t v : vs)
    for (int32_t r : rs) {
      int32_t c = 0, e = 0;
      EXPECT(whiflash_argmax_sweep_plan(r, v, &c, &e) == WF_OK, "plan");
      EXPECT(e % 256 == 0 && c >= 1, "plan chunk");
      EXPECT(int64_t(c) * e >= v && int64_t(c - 1) * e < v, "plan cover");
    }
  int32_t c = 0, e = 0;
  EXPECT(whiflash_argmax_sweep_plan(0, V, &c, &e) == WF_ERR_SHAPE, "plan rows 0");
  EXPECT(whiflash_argmax_sweep_plan(5, V, nullptr, &e) == WF_ERR_NULL, "plan null");
}

void workspace_sizes() {
  const int32_t ext[] = {-1, 0, 1, 2, 17, 1023, 1024, 65535, 65536, INT32_MAX / 8, INT32_MAX};
  for (int32_t a : ext)
    for (int32_t b : ext) {
      (void)whiflash_route_workspace_bytes(a, b);
      (void)whiflash_verify_workspace_bytes(a, b > 0 ? V : b);
      (void)whiflash_entropy_workspace_bytes(a, b);
      (void)whiflash_early_exit_workspace_bytes(a, b % 1024, V);
      (void)whiflash_tree_early_exit_workspace_bytes(a, b % 1025, V);
      (void)whiflash_round_workspace_bytes(a, b, a, V);
      (void)whiflash_round_chain_workspace_bytes(a, b, b % 1024, V);
      (void)whiflash_round_chain_early_exit_workspace_bytes(a, b, b % 1024, V);
      (void)whiflash_routed_early_exit_workspace_bytes(a, 16, 61, b, V);
      (void)whiflash_round_early_exit_workspace_bytes(a, 1024, 16, 61, b, V);
      (void)whiflash_verify_routed_entropy_workspace_bytes(a, b, V);
    }
  EXPECT(whiflash_route_workspace_bytes(256, 1024) % 256 == 0, "route ws align");
  EXPECT(whiflash_verify_workspace_bytes(4352, V) >= size_t(4352) * 8, "verify ws");
  EXPECT(whiflash_round_chain_workspace_bytes(INT32_MAX, 1024, 1023, V) == 0, "rows overflow");
}

void calls() {
  const float* f = static_cast<const float*>(A);
  const int32_t* i = static_cast<const int32_t*>(A);
  float* fo = static_cast<float*>(const_cast<void*>(A));
  int32_t* io = static_cast<int32_t*>(const_cast<void*>(A));
  struct Shape {
    int32_t B, K, N, d, m, dt;
  };
  const Shape shapes[] = {{1, 16, 61, 2560, 1024, WF_F32}, {5, 16, 61, 256, 64, WF_BF16},
                          {9, 0, 1, 96, 50, WF_BF16},      {32, 16, 61, 2560, 1024, WF_BF16},
                          {256, 16, 61, 2560, 320, WF_BF16}, {250, 1023, 1024, 104, 70, WF_BF16}};
  for (const Shape& s : shapes) {
    const int32_t crow = s.B * (s.K + 1), trow = s.B * s.N;
    char tag[96];
    snprintf(tag, sizeof tag, "B=%d K=%d N=%d d=%d m=%d dt=%d", s.B, s.K, s.N, s.d, s.m, s.dt);

    g_launches.clear();
    EXPECT(whiflash_route(A, s.dt, s.B, s.d, A, f, s.m, A, f, 1.f, fo, io, W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);
    g_launches.clear();
    EXPECT(whiflash_route(A, s.dt, s.B, WHIFLASH_MAX_HIDDEN, A, f, 1, A, f, 1.f, fo, io, W, kBig,
                          0) == WF_OK, tag);
    check_shapes(tag);
    check_per_sequence(tag, "router_finish_kernel", s.B);

    g_launches.clear();
    EXPECT(whiflash_verify_chain(A, s.dt, s.B, s.K, V, V, i, io, io, io, W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);
    check_sweep(tag, crow, V);
    check_per_sequence(tag, "finalize_chain_kernel", s.B);

    g_launches.clear();
    EXPECT(whiflash_verify_tree(A, s.dt, s.B, s.N, V, V, i, i, i, 32000, io, io, io, io, W, kBig,
                                0) == WF_OK, tag);
    check_shapes(tag);
    check_sweep(tag, trow, V);
    check_per_sequence(tag, "finalize_tree_kernel", s.B);

    g_launches.clear();
    EXPECT(whiflash_verify_routed(A, s.dt, s.B, V, V, i, trow, i, s.K, i, s.N, i, i, i, 32000, io,
                                  io, io, io, W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);
    check_sweep(tag, trow, V);
    check_per_sequence(tag, "finalize_routed_kernel", s.B);

    g_launches.clear();
    EXPECT(whiflash_round_chain(A, s.dt, s.d, A, f, s.m, A, f, 1.f, fo, io, A, s.dt, s.B, s.K, V,
                                V, i, io, io, io, W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);
    check_per_sequence(tag, "round_chain_finalize_kernel", s.B);

    g_launches.clear();
    EXPECT(whiflash_round_chain_noalloc(A, s.dt, s.d, A, f, s.m, A, f, 1.f, fo, io, A, s.dt, s.B,
                                        s.K, V, V, i, io, io, io, 0) ==
               (whiflash_round_chain_workspace_bytes(s.B, s.m, s.K, V) <=
                        WHIFLASH_NOALLOC_SCRATCH_BYTES
                    ? WF_OK
                    : WF_ERR_SCRATCH),
           tag);

    g_launches.clear();
    EXPECT(whiflash_round_routed(A, s.dt, s.d, A, f, s.m, A, f, 1.f, fo, io, A, s.dt, s.B, V, V,
                                 i, trow, s.K, i, s.N, i, i, i, 32000, io, io, io, io, W, kBig,
                                 0) == WF_OK, tag);
    check_shapes(tag);
    check_per_sequence(tag, "round_finalize_kernel", s.B);

    g_launches.clear();
    EXPECT(whiflash_verify_chain_early_exit(A, s.dt, s.B, s.K, V, V, i, io, io, io, W, kBig, 0) ==
               WF_OK, tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_verify_tree_early_exit(A, s.dt, s.B, s.N, V, V, i, i, i, 32000, io, io, io,
                                           io, W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_verify_routed_early_exit(A, s.dt, s.B, V, V, i, trow, i, s.K, i, s.N, i, i, i,
                                             32000, io, io, io, io, W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_round_routed_early_exit(A, s.dt, s.d, A, f, s.m, A, f, 1.f, fo, io, A, s.dt,
                                            s.B, V, V, i, trow, s.K, i, s.N, i, i, i, 32000, io,
                                            io, io, io, W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_round_chain_early_exit(A, s.dt, s.d, A, f, s.m, A, f, 1.f, fo, io, A, s.dt,
                                           s.B, s.K, V, V, i, io, io, io, W, kBig, 0) == WF_OK,
           tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_verify_routed_entropy(A, s.dt, s.B, V, V, i, trow, i, s.K, i, s.N, i, i, i,
                                          32000, 3.f, io, io, io, io, fo, io, W, kBig, 0) == WF_OK,
           tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_route_entropy(A, s.dt, trow, V, V, s.B, i, 0, i, 3.f, fo, io, W, kBig, 0) ==
               WF_OK, tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_route_gather(A, s.dt, trow, s.d, s.B, i, 0, i, A, f, s.m, A, f, 1.f, fo, io,
                                 W, kBig, 0) == WF_OK, tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_catchup_update(s.B, i, i, i, io, io, io, 0) == WF_OK, tag);
    check_shapes(tag);

    g_launches.clear();
    EXPECT(whiflash_argmax_sweep(A, s.dt, crow, V, V, W, kBig, 0) == WF_OK, tag);
    check_sweep(tag, crow, V, true);
    g_launches.clear();
    uint32_t* sink = static_cast<uint32_t*>(const_cast<void*>(A));
    EXPECT(whiflash_stream_read(A, s.dt, crow, V, V, sink, 0) == WF_OK, tag);
    check_shapes(tag);
  }
  EXPECT(has("stream_read_kernel"), "stream read launched");
}

void rejections() {
  const float* f = static_cast<const float*>(A);
  const int32_t* i = static_cast<const int32_t*>(A);
  float* fo = static_cast<float*>(const_cast<void*>(A));
  int32_t* io = static_cast<int32_t*>(const_cast<void*>(A));
  g_launches.clear();
  // Bad sizes, types, pointers, alignment and workspaces: a status, and nothing launched.
  EXPECT(whiflash_route(A, 7, 4, 64, A, f, 8, A, f, 1.f, fo, io, W, kBig, 0) == WF_ERR_DTYPE, "dt");
  EXPECT(whiflash_route(A, 1, 4, 0, A, f, 8, A, f, 1.f, fo, io, W, kBig, 0) == WF_ERR_SHAPE, "d");
  EXPECT(whiflash_route(A, 1, 65536, 64, A, f, 8, A, f, 1.f, fo, io, W, kBig, 0) == WF_ERR_SHAPE,
         "B");
  EXPECT(whiflash_route(A, 1, 4, 64, A, f, INT32_MAX, A, f, 1.f, fo, io, W, kBig, 0) ==
             WF_ERR_SHAPE, "m");
  EXPECT(whiflash_route(A, 1, 16, INT32_MAX - 7, A, f, 1, A, f, 1.f, fo, io, W, kBig, 0) ==
             WF_ERR_SHAPE, "d past the hidden-size limit");
  EXPECT(whiflash_verify_chain(A, 1, INT32_MAX, 1023, V, V, i, io, io, io, W, kBig, 0) ==
             WF_ERR_SHAPE, "rows overflow");
  EXPECT(whiflash_verify_chain(A, WF_F32, 4, 16, V, INT64_MAX / 2, i, io, io, io, W, kBig, 0) ==
             WF_ERR_SHAPE, "row stride whose byte size overflows");
  EXPECT(whiflash_verify_chain(A, WF_BF16, 4, 16, V, INT64_MAX, i, io, io, io, W, kBig, 0) ==
             WF_ERR_SHAPE, "row stride whose byte size overflows");
  EXPECT(whiflash_verify_tree(A, 1, 4, 61, V, V, i, i, i, 0, io, io, io, io, W, kBig, 0) ==
             WF_ERR_SHAPE, "Vd");
  EXPECT(whiflash_verify_routed(A, 1, 4, V, V, i, -1, i, 16, i, 61, i, i, i, 32000, io, io, io, io,
                                W, kBig, 0) == WF_ERR_SHAPE, "total_rows");
  EXPECT(whiflash_round_chain(A, 1, 2560, A, f, 1024, A, f, 1.f, fo, io, A, 1, 256, 16, V, V, i,
                              io, io, io, W, 64, 0) == WF_ERR_WORKSPACE, "ws small");
  EXPECT(whiflash_round_chain_noalloc(A, 1, 2560, A, f, 1024, A, f, 1.f, fo, io, A, 1, 1600, 16,
                                      V, V, i, io, io, io, 0) == WF_ERR_SCRATCH, "scratch");
  EXPECT(whiflash_argmax_sweep(static_cast<const char*>(A) + 4, 1, 8, V, V, W, kBig, 0) ==
             WF_ERR_ALIGN, "align");
  EXPECT(whiflash_catchup_update(-1, i, i, i, io, io, io, 0) != WF_OK, "catchup B");
  EXPECT(g_launches.empty(), "a rejected call launched a kernel");
  for (int32_t s = -9; s <= 1; ++s) EXPECT(whiflash_status_string(s) != nullptr, "status string");
}

// The interleaved numbering of a shared router + sweep launch (interleave.h) is a
// bijection onto the sweep's chunks and the router tiles, every XCD sweeps one
// contiguous range of chunks in increasing order, and every XCD runs r tiles.
void interleave_bijection() {
  const int64_t sweeps[] = {1, 7, 8, 9, 100, 2176, 5368, 5984, 8160, 47872, 65280, 74880};
  const int64_t routers[] = {1, 2, 3, 16, 32, 64, 128, 257};
  const int percents[] = {1, 25, 50, 75, 100};
  for (int64_t S : sweeps)
    for (int64_t r : routers)
      for (int pct : percents) {
        if (S / 8 < r) continue;  // the launch path requires a full set of router positions
        const int64_t n = S + 8 * r;
        const int64_t sp = wf::interleave_spacing(n, r, pct);
        char tag[96];
        snprintf(tag, sizeof tag, "interleave S=%lld r=%lld pct=%d", (long long)S, (long long)r, pct);
        EXPECT(sp >= 1 && r * sp <= n / 8, tag);
        std::vector<char> chunk(S, 0), tile(8 * r, 0);
        std::vector<int64_t> last(8, -1), lo(8, INT64_MAX), hi(8, -1), tiles_on(8, 0);
        for (int64_t i = 0; i < n; ++i) {
          const int64_t t = wf::interleave_map(i, n, r, sp);
          const int x = static_cast<int>(i % 8);
          if (t >= 0) {
            EXPECT(t < S && !chunk[t], tag);
            if (t < S) chunk[t] = 1;
            EXPECT(t > last[x], tag);  // increasing along the XCD's positions
            last[x] = t;
            lo[x] = t < lo[x] ? t : lo[x];
            hi[x] = t > hi[x] ? t : hi[x];
          } else {
            const int64_t u = -t - 1;
            EXPECT(u < 8 * r && !tile[u] && u / r == x, tag);
            if (u < 8 * r) tile[u] = 1;
            ++tiles_on[x];
          }
        }
        int64_t covered = 0;
        for (int x = 0; x < 8; ++x) {
          EXPECT(tiles_on[x] == r, tag);
          if (hi[x] >= 0) covered += hi[x] - lo[x] + 1;
          if (x > 0 && hi[x] >= 0 && hi[x - 1] >= 0) EXPECT(lo[x] == hi[x - 1] + 1, tag);
        }
        EXPECT(covered == S, tag);  // contiguous per XCD, no gaps or overlaps
      }
}

}  // namespace

int main() {
  interleave_bijection();
  plans();
  workspace_sizes();
  calls();
  rejections();
  if (g_failures) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("abi_driver: all checks passed\n");
  return 0;
}
