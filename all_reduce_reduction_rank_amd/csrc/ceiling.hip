// ceiling.hip -- streaming kernels that measure the practical HBM ceiling of
// this GPU for a given mix of reads and writes.  A measurement aid, not part
// of any collective: the collectives are streaming reductions bound by HBM
// bandwidth ("Collective communication: NCCL's algorithms and protocols, and
// custom all-reduce", section "Reading nccl-tests": bus bandwidth is read
// against the hardware's own bandwidth), and the fraction of the published
// 8 TB/s they reach is only meaningful next to what a pure stream with the
// same read:write mix reaches on the same GPU.
//
// stream_kernel<R, W>: R source streams and W destination streams of
// `bytes` each.  Every thread walks 16-byte vectors grid-stride; per vector it
// loads the vector of every source, combines them (exclusive or), and stores
// the result to every destination.  With W = 0 nothing is stored (a word that
// depends on every load keeps them live); with R = 0 each vector stored is
// made from its index.  Loads and stores are plain or non-temporal (as the
// collectives' once-touched data are), by the caller's choice.  Buffer
// resources bound every access.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/ar.h"
#include "device.hpp"

namespace {

constexpr int CEIL_MAX_READ = 8;
constexpr int CEIL_MAX_WRITE = 2;
constexpr int CEIL_THREADS = 256;

struct CeilArgs {
  const char* src[CEIL_MAX_READ];
  char* dst[CEIL_MAX_WRITE];
  uint64_t bytes;  // per stream, a multiple of 16
  uint32_t* sink;  // W = 0: one word
  int32_t load_policy, store_policy;  // buffer cache policy bits of the loads / stores
};

// Vectors per thread per stream in flight: UNROLL for one or two sources,
// else about 2*UNROLL loads per thread spread over the sources.
template <int R, int UNROLL>
constexpr int ceil_unroll() {
  return R <= 2 ? UNROLL : (2 * UNROLL / R < 1 ? 1 : 2 * UNROLL / R);
}

constexpr int CPOL_NT = 2;  // buffer-instruction cache policy: non-temporal

template <int R, int W, int UNROLL>
__global__ __launch_bounds__(CEIL_THREADS) void stream_kernel(CeilArgs a) {
  constexpr int U = ceil_unroll<R, UNROLL>();
  using namespace ar;
  const uint64_t nvec = a.bytes / 16;
  const uint64_t stride = (uint64_t)gridDim.x * CEIL_THREADS;
  // Buffer resources over each stream: a lane past the end reads zeros and
  // its store is dropped, so no per-lane branch separates the loads.
  Rsrc rs[R > 0 ? R : 1], rd[W > 0 ? W : 1];
#pragma unroll
  for (int r = 0; r < R; ++r) rs[r] = make_rsrc(a.src[r], (uint32_t)a.bytes);
#pragma unroll
  for (int w = 0; w < W; ++w) rd[w] = make_rsrc(a.dst[w], (uint32_t)a.bytes);
  uint32_t live = 0;
  for (uint64_t base = (uint64_t)blockIdx.x * CEIL_THREADS + threadIdx.x; base < nvec; base += stride * U) {
    uint4 x[U][R > 0 ? R : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t v = base + (uint64_t)u * stride;
      const uint32_t off = v < nvec ? (uint32_t)(v * 16) : 0xfffffff0u;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const v4u32 y = a.load_policy ? __builtin_amdgcn_raw_buffer_load_b128(rs[r], off, 0, CPOL_NT)
                                      : __builtin_amdgcn_raw_buffer_load_b128(rs[r], off, 0, 0);
        x[u][r] = make_uint4(y.x, y.y, y.z, y.w);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the pass is issued before any use
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t v = base + (uint64_t)u * stride;
      const uint32_t off = v < nvec ? (uint32_t)(v * 16) : 0xfffffff0u;
      uint4 acc = R == 0 ? make_uint4((uint32_t)v, (uint32_t)u, 0, 1) : x[u][0];
#pragma unroll
      for (int r = 1; r < R; ++r) {
        acc.x ^= x[u][r].x; acc.y ^= x[u][r].y; acc.z ^= x[u][r].z; acc.w ^= x[u][r].w;
      }
      const v4u32 y = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
      for (int w = 0; w < W; ++w) {
        if (a.store_policy) __builtin_amdgcn_raw_buffer_store_b128(y, rd[w], off, 0, CPOL_NT);
        else __builtin_amdgcn_raw_buffer_store_b128(y, rd[w], off, 0, 0);
      }
      if (W == 0) live ^= acc.x ^ acc.y ^ acc.z ^ acc.w;
    }
  }
  if (W == 0 && live == 0x9e3779b9u) a.sink[0] = live;  // keeps the loads live; practically never stores
}

using CeilFn = void (*)(CeilArgs);

template <int R, int W>
CeilFn pick_u(int u) {
  switch (u) {
    case 4: return stream_kernel<R, W, 4>;
    case 8: return stream_kernel<R, W, 8>;
    case 16: return stream_kernel<R, W, 16>;
    default: return nullptr;
  }
}

template <int R>
CeilFn pick_w(int w, int u) {
  switch (w) {
    case 0: return pick_u<R, 0>(u);
    case 1: return pick_u<R, 1>(u);
    case 2: return pick_u<R, 2>(u);
    default: return nullptr;
  }
}

CeilFn pick(int r, int w, int u) {
  switch (r) {
    case 0: return w ? pick_w<0>(w, u) : nullptr;
    case 1: return pick_w<1>(w, u);
    case 2: return pick_w<2>(w, u);
    case 3: return pick_w<3>(w, u);
    case 4: return pick_w<4>(w, u);
    case 5: return pick_w<5>(w, u);
    case 6: return pick_w<6>(w, u);
    case 7: return pick_w<7>(w, u);
    case 8: return pick_w<8>(w, u);
    default: return nullptr;
  }
}

// Workgroups of kernel f that fit on one CU, times the CUs, cached per
// (kernel, device).
int ceiling_grid(CeilFn f, int device, int* cus_out) {
  struct Entry { CeilFn f; int device, per_cu, cus; };
  static std::mutex mu;
  static Entry seen[128];
  static int used = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (seen[i].f == f && seen[i].device == device) {
      *cus_out = seen[i].cus;
      return seen[i].per_cu;
    }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)f, CEIL_THREADS, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) cus = 1;
  if (used < 128) seen[used++] = {f, device, per_cu, cus};
  *cus_out = cus;
  return per_cu;
}

}  // namespace

extern "C" ar_status ar_stream_ceiling(int nread, const void* const* src, int nwrite, void* const* dst, size_t bytes,
                                       void* sink, int flags, int unroll, int wg_per_cu, ar_stream_t stream) {
  if (flags & ~3) return AR_ERR_INVALID;
  if (unroll != 4 && unroll != 8 && unroll != 16) return AR_ERR_INVALID;
  if (wg_per_cu < 0) return AR_ERR_INVALID;
  if (nread < 0 || nread > CEIL_MAX_READ || nwrite < 0 || nwrite > CEIL_MAX_WRITE || nread + nwrite == 0)
    return AR_ERR_INVALID;
  if (bytes % 16 || bytes > (2ull << 30)) return AR_ERR_INVALID;
  if (nread && !src) return AR_ERR_INVALID;
  if (nwrite && !dst) return AR_ERR_INVALID;
  CeilArgs a = {};
  for (int r = 0; r < nread; ++r) {
    if (!src[r] || ((uintptr_t)src[r] & 15)) return AR_ERR_INVALID;
    a.src[r] = (const char*)src[r];
  }
  for (int w = 0; w < nwrite; ++w) {
    if (!dst[w] || ((uintptr_t)dst[w] & 15)) return AR_ERR_INVALID;
    a.dst[w] = (char*)dst[w];
  }
  if (nwrite == 0 && !sink) return AR_ERR_INVALID;
  a.bytes = bytes;
  a.sink = (uint32_t*)sink;
  a.load_policy = (flags & 1) ? CPOL_NT : 0;
  a.store_policy = (flags & 2) ? CPOL_NT : 0;
  if (bytes == 0) return AR_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AR_ERR_HIP;
  CeilFn f = pick(nread, nwrite, unroll);
  if (!f) return AR_ERR_INVALID;
  const uint64_t want = (bytes / 16 + CEIL_THREADS - 1) / CEIL_THREADS;
  int cus = 1;
  int per_cu = ceiling_grid(f, dev, &cus);
  if (wg_per_cu && wg_per_cu < per_cu) per_cu = wg_per_cu;
  uint64_t grid = (uint64_t)per_cu * (uint64_t)cus;
  if (want < grid) grid = want ? want : 1;
  hipLaunchKernelGGL(f, dim3((unsigned)grid), dim3(CEIL_THREADS), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}
