// call.hpp -- what the C ABI's collective entry points share: argument
// checks and planning of one call, and the kernel launches (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ar.h"
#include "device.hpp"
#include "plan.hpp"

namespace ar {

// Check the arguments of one collective call of `op` over `n` ranks and plan
// it.  Nothing is touched on the device and no HIP call is made.  AUTO
// choices are resolved (LL / LL128 only when the message fits
// `max_line_bytes`); `max_bytes` caps the larger of a rank's send and
// receive buffers.  On AR_OK *out is the call's geometry; out->ntasks == 0
// means there is nothing to launch (count 0, or an in-place single rank).
// Workspace limits (flags, line staging) are the caller's to check.
ar_status plan_call(int op, int n, const void* const* send, void* const* recv, uint64_t count, int dtype,
                    int algo, int proto, uint64_t chunk_bytes, uint64_t max_bytes, uint64_t max_line_bytes,
                    const Tuning& tune, Geometry* out);

// How a call was launched (for the call log and AR_DEBUG).
struct LaunchInfo {
  uint32_t grid = 0, batch = 0, counter_free = 0, by_die = 0;
};

hipError_t launch_collective(const KArgs& a, int device, hipStream_t stream, uint32_t max_workgroups,
                             LaunchInfo* info = nullptr);

// AR_DEBUG is set in the environment (read once).
bool debug_enabled();
hipError_t launch_reset(Ctl* c, hipStream_t stream);

}  // namespace ar
