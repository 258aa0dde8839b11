// noalloc.hip -- ar_allreduce_noalloc: the all-reduce of ar_allreduce for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// A communicator's workspace comes from one hipMalloc at creation.  Here the
// kernels' scratch (control block and Simple flags) lives instead in a
// file-scope device array of a fixed size, one copy per GPU, which the
// library holds until the process ends.  The call itself allocates nothing:
// no hipMalloc, no hipFree, no library routine that allocates.
//
// The array's name is a host-side stand-in, not a device address.  On the
// first call on a device, with that device current, hipGetSymbolAddress
// yields the address of that device's copy; it is kept per device and is the
// only handle host code ever passes on (kernel arguments, the clearing
// kernel).
//
// Every call on a GPU shares its copy, which keeps the last call's contents:
//   - the first call on a device clears the whole array (a fill kernel on the
//     caller's stream, ahead of its collective);
//   - flags are tagged with the call counter kept in the array, so they are
//     never cleared again (as in a communicator's workspace);
//   - the ticket and exit counters, the abort word and the error record must
//     be zero (the error key all ones) when a call starts: the last workgroup
//     out of every call re-arms them.
// Calls that overlap on one GPU (two streams, or a graph replayed beside an
// eager call) race on the array: the caller must order them.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "call.hpp"
#include "calllog.hpp"

using namespace ar;

namespace {

constexpr uint64_t SCRATCH_BYTES = 8ull << 20;  // control block + Simple flags
constexpr uint64_t CTL_BYTES = (sizeof(Ctl) + 255) & ~255ull;
constexpr uint64_t SCRATCH_FLAGS = (SCRATCH_BYTES - CTL_BYTES) / 8;
constexpr uint64_t MAX_RANK_BYTES = 1ull << 30;  // at most 1 GiB per rank
constexpr int MAX_DEVICES = 64;
static_assert(offsetof(Ctl, err_key) % 8 == 0, "the error key starts an 8-byte word");

}  // namespace

static __device__ __align__(256) uint64_t scratch[SCRATCH_BYTES / 8];

// Clears the array: zeros everywhere, except the error key (all ones: no
// blocked wait recorded).
__global__ void scratch_clear_kernel(uint64_t* p, uint64_t nwords, uint64_t key_word) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < nwords;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = (i == key_word) ? 0xffffffffull : 0ull;
}

namespace {

struct DeviceScratch {
  uint64_t* ptr = nullptr;    // this device's copy of `scratch`
  uint64_t ticks_per_us = 100;
};

std::mutex g_mu;
DeviceScratch g_dev[MAX_DEVICES];

// Set-up on the first call on `dev` (the current device): the address of
// its copy of the array, the wall-clock rate for the waits' time limit, and
// one clear of the array on `stream`.
ar_status device_scratch(int dev, hipStream_t stream, DeviceScratch* out) {
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return AR_ERR_HIP;
    }
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz >= 1000)
      d.ticks_per_us = (uint64_t)khz / 1000;
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(256), dim3(256), 0, stream, (uint64_t*)p, SCRATCH_BYTES / 8,
                       (uint64_t)(offsetof(Ctl, err_key) / 8));
    if (hipGetLastError() != hipSuccess) return AR_ERR_HIP;
    d.ptr = (uint64_t*)p;
  }
  *out = d;
  return AR_OK;
}

}  // namespace

extern "C" ar_status ar_allreduce_noalloc(int nranks, const void* const* send, void* const* recv, size_t count,
                                          ar_dtype dtype, ar_algo algo, ar_proto proto, size_t chunk_bytes,
                                          ar_stream_t stream) {
  if (nranks < 1 || nranks > MAX_RANKS) return AR_ERR_INVALID;
  // Line staging grows with the message: only Simple runs from the array.
  if ((int)proto == PROTO_LL || (int)proto == PROTO_LL128) return AR_ERR_UNSUPPORTED;
  Geometry g;
  const ar_status st = plan_call(OP_ALLREDUCE, nranks, send, recv, count, (int)dtype, (int)algo, (int)proto,
                                 chunk_bytes, MAX_RANK_BYTES, 0, Tuning(), &g);
  if (st != AR_OK || g.ntasks == 0) return st;
  if (g.nflags > SCRATCH_FLAGS) return AR_ERR_TOO_LARGE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return AR_ERR_HIP;
  DeviceScratch d;
  const ar_status sst = device_scratch(dev, (hipStream_t)stream, &d);
  if (sst != AR_OK) return sst;

  KArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < nranks; ++r) {
    a.in[r] = (const char*)send[r];
    a.out[r] = (char*)recv[r];
  }
  a.g = g;
  a.ctl = (Ctl*)d.ptr;
  a.flags = d.ptr + CTL_BYTES / 8;
  a.lines = nullptr;  // Simple only
  a.stage = nullptr;  // all-reduce: no reduce-scatter partials
  a.timeout = 5ull * 1000 * 1000 * d.ticks_per_us;  // 5 s
  a.inj_rank = -1;
  a.inj_step = -1;
  a.rearm_errors = 1;
  LaunchInfo info;
  if (launch_collective(a, dev, (hipStream_t)stream, 0, &info) != hipSuccess) return AR_ERR_HIP;
  if (debug_enabled()) {
    ar_call_record r = {};
    r.op = OP_ALLREDUCE;
    r.algo = g.algo;
    r.proto = g.proto;
    r.dtype = g.dtype;
    r.nranks = g.nranks;
    r.in_place = g.in_place;
    r.grid = info.grid;
    r.batch = info.batch;
    r.counter_free = info.counter_free;
    r.by_die = info.by_die;
    r.count = count;
    r.ntasks = g.ntasks;
    r.tile_bytes = g.tile * (uint64_t)g.esize;
    char line[320];
    format_record(line, sizeof(line), r);
    fprintf(stderr, "[ar] noalloc %s\n", line);
  }
  return AR_OK;
}
