// rmsnorm.hpp -- arguments of the fused all-reduce + RMSNorm kernel
// (rmsnorm.hip), shared with the C ABI (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.hpp"

namespace ar {

constexpr uint64_t RMS_MAX_HIDDEN = 12288;  // a row's fp32 h in registers: 48 floats per thread

struct RmsArgs {
  const char* in[MAX_RANKS];
  char* out[MAX_RANKS];
  char* res[MAX_RANKS];  // nullptr: no residual
  const char* weight;
  uint64_t rows, hidden;  // hidden: a multiple of one 16-byte vector
  int32_t nranks;
  float eps;
  uint32_t by_die;  // N > 0: the N items of each row run on one die (die_ticket)
};

hipError_t launch_rmsnorm(const RmsArgs& a, int dtype, int device, hipStream_t stream, uint32_t max_workgroups);

}  // namespace ar
