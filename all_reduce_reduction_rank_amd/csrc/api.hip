// api.hip -- the C ABI declared in include/ar.h.
//
// A communicator ("Add nccl support for tensor parrallel", overview: a
// communicator is set up once, then collective calls are made on it) owns one
// device workspace allocated at creation, as a custom all-reduce's
// pre-registered buffer is ("Collective communication: NCCL's algorithms and
// protocols, and custom all-reduce", exercise 3): calls allocate nothing, so
// they can be captured in HIP graphs, and the workspace caps the message size.
//
// Workspace layout (one hipMalloc, 256-byte aligned regions):
//   [Ctl][flags: u64 x nflags][LL lines][LL128 lines][ring reduce-scatter partials]
// Ctl, flags and lines are zeroed at creation; flags and lines are tagged
// with the device call counter, so they are never cleared again.
// LL and LL128 stage in separate regions, as NCCL keeps a buffer per
// protocol.  An LL reader takes bytes 4-7 of every 8-byte slot as a flag;
// in a shared region those bytes can hold an earlier LL128 call's payload,
// and a payload word that equals the current LL flag would pass a stale line
// as fresh.  In its own region an LL flag slot only ever holds an LL flag of
// this or an earlier call; LL128 flag words (bytes 120-127 of each line)
// likewise only ever hold LL128 flags.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/ar.h"
#include "device.hpp"
#include "plan.hpp"
#include "call.hpp"
#include "calllog.hpp"
#include "rmsnorm.hpp"

using namespace ar;

struct ar_comm {
  int nranks = 0;
  int device = 0;
  size_t max_bytes = 0, max_line_bytes = 0;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  Ctl* ctl = nullptr;
  uint64_t* flags = nullptr;
  uint64_t nflags = 0;
  char* lines[2] = {nullptr, nullptr};  // LL, LL128 staging
  uint64_t lines_bytes[2] = {0, 0};
  char* stage = nullptr;
  uint64_t stage_stride = 0;
  uint64_t ticks_per_us = 100;
  uint64_t timeout_ticks = 0;
  int inj_rank = -1, inj_step = -1;
  uint32_t max_workgroups = 0;  // 0: as many as fit on the GPU
  bool broken = false;
  CallLog log;                  // the most recent calls launched
};

static uint64_t align256(uint64_t x) { return (x + 255) & ~255ull; }

// Tuning overrides read once from the environment (for measurements; they
// never change results): AR_TILE_KB, AR_LINE_TILE_KB, AR_RING_SKEW,
// AR_RING_WINDOW, AR_LAG, AR_COLOC_TILE_KB.
static const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning x;
    if (const char* e = getenv("AR_TILE_KB")) x.tile_bytes = strtoull(e, nullptr, 10) * 1024;
    if (const char* e = getenv("AR_LINE_TILE_KB")) x.line_tile_bytes = strtoull(e, nullptr, 10) * 1024;
    if (const char* e = getenv("AR_RING_SKEW")) { x.ring_skew = strtoull(e, nullptr, 10); x.ring_skew_set = true; }
    if (const char* e = getenv("AR_RING_WINDOW")) x.ring_window = strtoull(e, nullptr, 10);
    if (const char* e = getenv("AR_LAG")) x.lag = strtoull(e, nullptr, 10);
    if (const char* e = getenv("AR_COLOC_TILE_KB")) {
      x.coloc_tile_bytes = strtoull(e, nullptr, 10) * 1024;
      x.coloc_tile_set = true;
    }
    return x;
  }();
  return t;
}

// Largest staging any call of protocol `proto` (LL or LL128) on payloads of
// up to `line_bytes` per rank can need (the ring all-reduce dominates;
// checked again per call).
static uint64_t line_capacity(int n, uint64_t line_bytes, int proto) {
  if (!line_bytes) return 0;
  uint64_t best = 0;
  for (int op = 0; op < 3; ++op)
    for (int algo = 0; algo < 3; ++algo)
      for (int dt = 0; dt < 3; dt += 1) {
        const uint64_t es = (uint64_t)esize_of(dt);
        const uint64_t cnt = op == OP_ALLREDUCE ? line_bytes / es : line_bytes / es / n;
        Geometry g;
        if (make_geometry(op, algo, proto, dt, n, cnt, 0, 0, &g)) best = umax(best, staging_bytes(g));
      }
  return best + best / 8 + (1u << 20);
}

extern "C" {

const char* ar_status_string(ar_status s) {
  switch (s) {
    case AR_OK: return "ok";
    case AR_ERR_INVALID: return "invalid argument";
    case AR_ERR_UNSUPPORTED: return "unsupported combination";
    case AR_ERR_NOMEM: return "out of device memory";
    case AR_ERR_TOO_LARGE: return "message exceeds the communicator's capacity";
    case AR_ERR_HIP: return "HIP runtime error";
    case AR_ERR_TIMEOUT: return "a rank program timed out waiting for a peer";
    case AR_ERR_BROKEN: return "communicator holds a latched device error";
  }
  return "unknown status";
}

ar_status ar_comm_create(int nranks, size_t max_bytes_per_rank, size_t max_line_bytes_per_rank,
                         ar_comm_t* out) {
  if (!out || nranks < 1 || nranks > MAX_RANKS) return AR_ERR_INVALID;
  *out = nullptr;
  ar_comm* c = new ar_comm();
  c->nranks = nranks;
  c->max_bytes = max_bytes_per_rank;
  c->max_line_bytes = max_line_bytes_per_rank;
  if (hipGetDevice(&c->device) != hipSuccess) { delete c; return AR_ERR_HIP; }
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, c->device) == hipSuccess && khz > 0)
    c->ticks_per_us = (uint64_t)khz / 1000 ? (uint64_t)khz / 1000 : 1;
  c->timeout_ticks = 5ull * 1000 * 1000 * c->ticks_per_us;  // 5 s

  const uint64_t n = (uint64_t)nranks;
  c->nflags = umax(65536, 2 * n * (max_bytes_per_rank / 4096 + 8));
  c->lines_bytes[0] = line_capacity(nranks, max_line_bytes_per_rank, PROTO_LL);
  c->lines_bytes[1] = line_capacity(nranks, max_line_bytes_per_rank, PROTO_LL128);
  c->stage_stride = align256(max_bytes_per_rank);
  const uint64_t off_flags = align256(sizeof(Ctl));
  const uint64_t off_ll = off_flags + align256(c->nflags * 8);
  const uint64_t off_ll128 = off_ll + align256(c->lines_bytes[0]);
  const uint64_t off_stage = off_ll128 + align256(c->lines_bytes[1]);
  c->ws_bytes = off_stage + (nranks > 1 ? n * c->stage_stride : 0);
  if (hipMalloc((void**)&c->ws, c->ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return AR_ERR_NOMEM;
  }
  c->ctl = (Ctl*)c->ws;
  c->flags = (uint64_t*)(c->ws + off_flags);
  c->lines[0] = c->ws + off_ll;
  c->lines[1] = c->ws + off_ll128;
  c->stage = c->ws + off_stage;
  Ctl init = {};
  init.err_key = 0xffffffffu;
  if (hipMemset(c->ws, 0, off_stage) != hipSuccess ||
      hipMemcpy(c->ctl, &init, sizeof(Ctl), hipMemcpyHostToDevice) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(c->ws);
    delete c;
    return AR_ERR_HIP;
  }
  *out = c;
  return AR_OK;
}

ar_status ar_comm_destroy(ar_comm_t c) {
  if (!c) return AR_ERR_INVALID;
  const hipError_t e = hipFree(c->ws);
  delete c;
  return e == hipSuccess ? AR_OK : AR_ERR_HIP;
}

size_t ar_comm_workspace_bytes(ar_comm_t c) { return c ? c->ws_bytes : 0; }

ar_status ar_comm_check(ar_comm_t c, ar_stream_t stream, int* err_rank, int* err_step) {
  if (!c) return AR_ERR_INVALID;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return AR_ERR_HIP;
  Ctl h;
  if (hipMemcpy(&h, c->ctl, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return AR_ERR_HIP;
  if (!h.err_code) return AR_OK;
  c->broken = true;
  if (debug_enabled()) {
    fprintf(stderr,
            "[ar] latched error %d: first blocked wait rank %d step %d; flag %llu held %llu, awaited %llu "
            "(call counter %llu); last calls:\n",
            (int)h.err_code, h.err_key == 0xffffffffu ? -1 : (int)(h.err_key & 0xff),
            h.err_key == 0xffffffffu ? -1 : (int)(h.err_key >> 8), (unsigned long long)h.diag[1],
            (unsigned long long)h.diag[2], (unsigned long long)h.diag[3], (unsigned long long)h.diag[4]);
    ar_call_record recs[CallLog::CAP];
    const int n = c->log.copy(recs, CallLog::CAP);
    for (int i = 0; i < n; ++i) {
      char line[320];
      format_record(line, sizeof(line), recs[i]);
      fprintf(stderr, "[ar]   %s\n", line);
    }
  }
  if (err_rank) *err_rank = h.err_key == 0xffffffffu ? -1 : (int)(h.err_key & 0xff);
  if (err_step) *err_step = h.err_key == 0xffffffffu ? -1 : (int)(h.err_key >> 8);
  return (ar_status)h.err_code;
}

ar_status ar_comm_set_max_workgroups(ar_comm_t c, unsigned max_workgroups) {
  if (!c) return AR_ERR_INVALID;
  c->max_workgroups = max_workgroups;
  return AR_OK;
}

ar_status ar_debug_state(ar_comm_t c, ar_stream_t stream, uint64_t* out, int n) {
  if (!c || !out || n < 0) return AR_ERR_INVALID;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return AR_ERR_HIP;
  Ctl h;
  if (hipMemcpy(&h, c->ctl, sizeof(Ctl), hipMemcpyDeviceToHost) != hipSuccess) return AR_ERR_HIP;
  const uint64_t words[10] = {h.diag[0], h.diag[1], h.diag[2], h.diag[3], h.diag[4], h.diag[5],
                              h.epoch, h.ticket, h.done, h.abort};
  for (int i = 0; i < n && i < 10; ++i) out[i] = words[i];
  return AR_OK;
}

ar_status ar_debug_calls(ar_comm_t c, ar_call_record* out, int max, int* n_out) {
  if (!c || !n_out || max < 0 || (max > 0 && !out)) return AR_ERR_INVALID;
  *n_out = c->log.copy(out, max);
  return AR_OK;
}

ar_status ar_comm_reset(ar_comm_t c, ar_stream_t stream) {
  if (!c) return AR_ERR_INVALID;
  if (ar::launch_reset(c->ctl, (hipStream_t)stream) != hipSuccess) return AR_ERR_HIP;
  c->broken = false;
  return AR_OK;
}

ar_status ar_debug_inject(ar_comm_t c, int rank, int step, uint64_t timeout_us) {
  if (!c || rank >= c->nranks || rank < -1) return AR_ERR_INVALID;
  c->inj_rank = rank;
  c->inj_step = rank < 0 ? -1 : step;
  c->timeout_ticks = (timeout_us ? timeout_us : 5ull * 1000 * 1000) * c->ticks_per_us;
  return AR_OK;
}

ar_status ar_select(int nranks, ar_op op, size_t count, ar_dtype dtype, ar_algo algo, ar_proto proto,
                    size_t max_line_bytes_per_rank, ar_algo* chosen_algo, ar_proto* chosen_proto,
                    double* predicted_us) {
  if (!chosen_algo || !chosen_proto) return AR_ERR_INVALID;
  if ((int)op < 0 || (int)op > 2 || (int)dtype < 0 || (int)dtype > 2) return AR_ERR_INVALID;
  if (nranks < 1 || nranks > MAX_RANKS) return AR_ERR_INVALID;
  const uint64_t es = (uint64_t)esize_of((int)dtype);
  const uint64_t in_bytes = ((int)op == OP_REDUCE_SCATTER ? (uint64_t)nranks * count : count) * es;
  const uint64_t out_bytes = ((int)op == OP_ALLGATHER ? (uint64_t)nranks * count : count) * es;
  const uint64_t rank_bytes = umax(in_bytes, out_bytes);
  int a = 0, p = 0;
  double t = -1.0;
  if (!select_schedule((int)op, nranks, (int)dtype, rank_bytes, (int)algo, (int)proto,
                       nranks > 1 && rank_bytes <= max_line_bytes_per_rank, &a, &p, &t))
    return AR_ERR_INVALID;
  *chosen_algo = (ar_algo)a;
  *chosen_proto = (ar_proto)p;
  if (predicted_us) *predicted_us = t;
  return AR_OK;
}

ar_status ar_plan_bytes(int nranks, ar_op op, size_t count, ar_dtype dtype, ar_algo algo, ar_proto proto,
                        size_t chunk_bytes, int in_place, uint64_t* hbm_read, uint64_t* hbm_write,
                        uint64_t* link_bytes, uint64_t* ntasks) {
  Geometry g;
  if (!make_geometry((int)op, (int)algo, (int)proto, (int)dtype, nranks, count, chunk_bytes, in_place, &g))
    return AR_ERR_INVALID;
  const Bytes b = account(g);
  if (hbm_read) *hbm_read = b.rd;
  if (hbm_write) *hbm_write = b.wr;
  if (link_bytes)
    for (int r = 0; r < nranks; ++r) link_bytes[r] = b.link[r];
  if (ntasks) *ntasks = g.ntasks;
  return AR_OK;
}

}  // extern "C"

// Do [a, a+na) and [b, b+nb) overlap?
static bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

ar_status ar::plan_call(int op, int n, const void* const* send, void* const* recv, uint64_t count, int dtype,
                        int algo, int proto, uint64_t chunk_bytes, uint64_t max_bytes, uint64_t max_line_bytes,
                        const Tuning& tune, Geometry* out) {
  memset(out, 0, sizeof(*out));
  if (!send || !recv) return AR_ERR_INVALID;
  if (dtype < 0 || dtype > 2 || algo < 0 || algo > ALGO_AUTO || proto < 0 || proto > PROTO_AUTO)
    return AR_ERR_INVALID;
  if (count == 0) return AR_OK;  // nothing to move; buffers may be null
  const uint64_t es = (uint64_t)esize_of(dtype);
  const uint64_t in_bytes = (op == OP_REDUCE_SCATTER ? (uint64_t)n * count : count) * es;
  const uint64_t out_bytes = (op == OP_ALLGATHER ? (uint64_t)n * count : count) * es;
  if (count > (1ull << 40)) return AR_ERR_TOO_LARGE;
  const uint64_t rank_bytes = umax(in_bytes, out_bytes);
  if (rank_bytes > max_bytes) return AR_ERR_TOO_LARGE;
  if (algo == ALGO_AUTO || proto == PROTO_AUTO) {
    const bool line_ok = n > 1 && rank_bytes <= max_line_bytes;
    if (!select_schedule(op, n, dtype, rank_bytes, algo, proto, line_ok, &algo, &proto, nullptr))
      return AR_ERR_INVALID;
  }
  if (algo == ALGO_TREE && n > 1 && (op != OP_ALLREDUCE || proto != PROTO_SIMPLE)) return AR_ERR_UNSUPPORTED;
  if (proto != PROTO_SIMPLE && n > 1 && rank_bytes > max_line_bytes) return AR_ERR_TOO_LARGE;

  int in_place = 0, same = 0;
  for (int r = 0; r < n; ++r) {
    if (!send[r] || !recv[r]) return AR_ERR_INVALID;
    if (((uintptr_t)send[r] & 15) || ((uintptr_t)recv[r] & 15)) return AR_ERR_INVALID;
    same += (send[r] == (const void*)recv[r]);
  }
  if (same == n && op == OP_ALLREDUCE) in_place = 1;
  else if (same) return AR_ERR_INVALID;  // partial in-place, or in-place RS / AG
  // Outputs must not overlap each other, nor (out of place) any input.
  for (int r = 0; r < n; ++r) {
    for (int q = 0; q < n; ++q) {
      if (q != r && overlap(recv[r], out_bytes, recv[q], out_bytes)) return AR_ERR_INVALID;
      if (!in_place && overlap(recv[r], out_bytes, send[q], in_bytes)) return AR_ERR_INVALID;
    }
  }
  if (!make_geometry(op, algo, proto, dtype, n, count, chunk_bytes, in_place, out, tune)) return AR_ERR_INVALID;
  if (out->ntasks >= (1ull << 31)) return AR_ERR_TOO_LARGE;
  return AR_OK;
}

static ar_status run(ar_comm_t c, int op, const void* const* send, void* const* recv, uint64_t count,
                     int dtype, int algo, int proto, uint64_t chunk_bytes, ar_stream_t stream) {
  if (!c || !send || !recv) return AR_ERR_INVALID;
  if (c->broken) return AR_ERR_BROKEN;
  if (dtype < 0 || dtype > 2 || algo < 0 || algo > ALGO_AUTO || proto < 0 || proto > PROTO_AUTO)
    return AR_ERR_INVALID;
  if (count == 0) return AR_OK;  // nothing to move; buffers may be null
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return AR_ERR_INVALID;
  Geometry g;
  const ar_status st = plan_call(op, c->nranks, send, recv, count, dtype, algo, proto, chunk_bytes, c->max_bytes,
                                 c->max_line_bytes, tuning(), &g);
  if (st != AR_OK || g.ntasks == 0) return st;
  const int li = g.proto == PROTO_LL128 ? 1 : 0;
  if (g.nflags > c->nflags || staging_bytes(g) > c->lines_bytes[li]) return AR_ERR_TOO_LARGE;

  KArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < c->nranks; ++r) {
    a.in[r] = (const char*)send[r];
    a.out[r] = (char*)recv[r];
  }
  a.g = g;
  a.ctl = c->ctl;
  a.flags = c->flags;
  a.lines = c->lines[li];
  a.stage = c->stage;
  a.stage_stride = c->stage_stride;
  a.timeout = c->timeout_ticks;
  a.inj_rank = c->inj_rank;
  a.inj_step = c->inj_step;
  LaunchInfo info;
  if (ar::launch_collective(a, c->device, (hipStream_t)stream, c->max_workgroups, &info) != hipSuccess)
    return AR_ERR_HIP;
  ar_call_record rec = {};
  rec.op = op;
  rec.algo = g.algo;
  rec.proto = g.proto;
  rec.dtype = g.dtype;
  rec.nranks = g.nranks;
  rec.in_place = g.in_place;
  rec.grid = info.grid;
  rec.batch = info.batch;
  rec.counter_free = info.counter_free;
  rec.by_die = info.by_die;
  rec.count = count;
  rec.ntasks = g.ntasks;
  rec.tile_bytes = g.tile * (uint64_t)g.esize;
  c->log.add(rec);
  if (debug_enabled()) {
    char line[320];
    format_record(line, sizeof(line), c->log.ring[(c->log.logged - 1) % CallLog::CAP]);
    fprintf(stderr, "[ar] %s\n", line);
  }
  return AR_OK;
}

extern "C" {

ar_status ar_allreduce(ar_comm_t c, const void* const* send, void* const* recv, size_t count, ar_dtype dtype,
                       ar_algo algo, ar_proto proto, size_t chunk_bytes, ar_stream_t stream) {
  return run(c, OP_ALLREDUCE, send, recv, count, dtype, algo, proto, chunk_bytes, stream);
}

ar_status ar_allreduce_rmsnorm(ar_comm_t c, const void* const* send, void* const* out, void* const* residual,
                               const void* weight, size_t rows, size_t hidden, float eps, ar_dtype dtype,
                               ar_stream_t stream) {
  if (!c || !send || !out) return AR_ERR_INVALID;
  if (c->broken) return AR_ERR_BROKEN;
  if ((int)dtype < 0 || (int)dtype > 2) return AR_ERR_INVALID;
  if (dtype == AR_I32) return AR_ERR_UNSUPPORTED;  // a norm of integers is not defined
  if (!(eps >= 0.0f) || eps > 3.0e38f) return AR_ERR_INVALID;
  if (rows == 0 || hidden == 0) return AR_OK;
  const uint64_t es = (uint64_t)esize_of((int)dtype);
  if ((hidden * es) % 16) return AR_ERR_INVALID;  // rows of whole 16-byte vectors
  if (hidden > RMS_MAX_HIDDEN) return AR_ERR_UNSUPPORTED;
  if (rows > (1ull << 40) / hidden) return AR_ERR_TOO_LARGE;
  const uint64_t bytes = (uint64_t)rows * hidden * es;
  if (bytes > c->max_bytes) return AR_ERR_TOO_LARGE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return AR_ERR_INVALID;
  if (!weight || ((uintptr_t)weight & 15)) return AR_ERR_INVALID;
  const int n = c->nranks;
  for (int r = 0; r < n; ++r) {
    if (!send[r] || !out[r] || ((uintptr_t)send[r] & 15) || ((uintptr_t)out[r] & 15)) return AR_ERR_INVALID;
    if (residual && (!residual[r] || ((uintptr_t)residual[r] & 15))) return AR_ERR_INVALID;
  }
  // Outputs and residuals are written: none may overlap another buffer.
  for (int r = 0; r < n; ++r) {
    if (overlap(out[r], bytes, weight, hidden * es)) return AR_ERR_INVALID;
    if (residual && overlap(residual[r], bytes, weight, hidden * es)) return AR_ERR_INVALID;
    for (int q = 0; q < n; ++q) {
      if (overlap(out[r], bytes, send[q], bytes)) return AR_ERR_INVALID;
      if (q != r && overlap(out[r], bytes, out[q], bytes)) return AR_ERR_INVALID;
      if (residual) {
        if (overlap(residual[r], bytes, send[q], bytes) || overlap(residual[r], bytes, out[q], bytes))
          return AR_ERR_INVALID;
        if (q != r && overlap(residual[r], bytes, residual[q], bytes)) return AR_ERR_INVALID;
      }
    }
  }
  RmsArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < n; ++r) {
    a.in[r] = (const char*)send[r];
    a.out[r] = (char*)out[r];
    a.res[r] = residual ? (char*)residual[r] : nullptr;
  }
  a.weight = (const char*)weight;
  a.rows = rows;
  a.hidden = hidden;
  a.nranks = n;
  a.eps = eps;
  return ar::launch_rmsnorm(a, (int)dtype, c->device, (hipStream_t)stream, c->max_workgroups) == hipSuccess
             ? AR_OK
             : AR_ERR_HIP;
}

ar_status ar_reduce_scatter(ar_comm_t c, const void* const* send, void* const* recv, size_t recvcount,
                            ar_dtype dtype, ar_algo algo, ar_proto proto, size_t chunk_bytes,
                            ar_stream_t stream) {
  return run(c, OP_REDUCE_SCATTER, send, recv, recvcount, dtype, algo, proto, chunk_bytes, stream);
}

ar_status ar_allgather(ar_comm_t c, const void* const* send, void* const* recv, size_t sendcount,
                       ar_dtype dtype, ar_algo algo, ar_proto proto, size_t chunk_bytes, ar_stream_t stream) {
  return run(c, OP_ALLGATHER, send, recv, sendcount, dtype, algo, proto, chunk_bytes, stream);
}

}  // extern "C"
