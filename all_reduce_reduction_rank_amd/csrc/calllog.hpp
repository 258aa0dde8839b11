// calllog.hpp -- a communicator's log of its most recent calls, and the
// one-line text of a call's plan printed when AR_DEBUG is set.  Pure C++
// (no HIP): the log lives on the host, beside the communicator.
//
// "Collective communication: NCCL's algorithms and protocols, and custom
// all-reduce", section "Common environment variables and debugging": the
// library's debug output names the schedules it built, and a flight recorder
// keeps each rank's recent collectives so that a hang can be traced back to
// the call a rank missed.  Here one communicator runs every rank, so one log
// holds the calls of all of them.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include "../../include/ar.h"

namespace ar {

struct CallLog {
  static constexpr int CAP = 16;  // calls kept
  ar_call_record ring[CAP] = {};
  uint64_t logged = 0;            // calls ever logged

  void add(ar_call_record r) {
    r.seq = ++logged;
    ring[(r.seq - 1) % CAP] = r;
  }
  // The most recent min(max, kept) calls, oldest first; returns how many.
  int copy(ar_call_record* out, int max) const {
    const uint64_t kept = logged < (uint64_t)CAP ? logged : (uint64_t)CAP;
    const int n = max < 0 ? 0 : ((uint64_t)max < kept ? max : (int)kept);
    for (int i = 0; i < n; ++i) out[i] = ring[(logged - (uint64_t)n + (uint64_t)i) % CAP];
    return n;
  }
};

inline const char* op_name(int op) {
  return op == 0 ? "allreduce" : op == 1 ? "reduce_scatter" : op == 2 ? "allgather" : "?";
}
inline const char* algo_name(int a) {
  return a == 0 ? "oneshot" : a == 1 ? "twoshot" : a == 2 ? "ring" : a == 3 ? "tree" : "?";
}
inline const char* proto_name(int p) { return p == 0 ? "simple" : p == 1 ? "ll" : p == 2 ? "ll128" : "?"; }
inline const char* dtype_name(int d) { return d == 0 ? "f32" : d == 1 ? "bf16" : d == 2 ? "i32" : "?"; }

// One line: "call 3: allreduce ring/simple f32 N=8 count=... out of place,
// tile 32768 B, 458752 tasks, grid 768 x batch 2".
inline int format_record(char* buf, size_t len, const ar_call_record& r) {
  return snprintf(buf, len,
                  "call %llu: %s %s/%s %s N=%d count=%llu %s, tile %llu B, %llu tasks, grid %u x batch %u%s%s",
                  (unsigned long long)r.seq, op_name(r.op), algo_name(r.algo), proto_name(r.proto),
                  dtype_name(r.dtype), r.nranks, (unsigned long long)r.count, r.in_place ? "in place" : "out of place",
                  (unsigned long long)r.tile_bytes, (unsigned long long)r.ntasks, r.grid, r.batch,
                  r.counter_free ? ", no ticket counter" : "", r.by_die ? ", by die" : "");
}

}  // namespace ar
