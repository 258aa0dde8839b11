// device.hpp -- payload arithmetic, memory access and rank-to-rank signalling
// for the gfx950 kernels.
//
// Arithmetic ("NCCL collectives, ring all-reduce & launching TP/PP", section
// "Direct answer": all-reduce sums): fp32 is one IEEE add per term (the build
// keeps denormals and has no contraction to apply, since there are only adds);
// int32 adds wrap; bf16 is widened exactly to fp32, added in fp32 and rounded
// to nearest even when stored or put on the wire.
//
// Signalling ("Collective communication: NCCL's algorithms and protocols, and
// custom all-reduce", section "Protocols").  The eight XCDs of an MI355X have
// private L2 caches, so data crossing rank programs uses device-scope (sc1)
// accesses, which bypass the XCD-private caching (see "device-coherent data
// accesses" below):
//   Simple  the producer stores its block with device-scope stores, waits for
//           them to complete, then stores a flag; the consumer polls the flag
//           with device-scope atomic loads, then reads with device-scope loads.
//   LL      each 8-byte line = 4 payload bytes + a 4-byte flag, written and
//           read as ONE 64-bit device-scope atomic: a reader that sees the
//           flag sees the payload.
//   LL128   each 128-byte line = 120 payload bytes + an 8-byte flag.  gfx950
//           gives no 128-byte single-copy atomicity, so the writer stores the
//           payload (device scope), waits for completion, then stores the
//           flag word; the reader polls the flag, then reads the payload
//           (device scope).  The byte layout (and so the 120/128 efficiency)
//           is the page's; the ordering is made explicit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.hpp"

namespace ar {

// ----------------------------------------------------------------- numerics
__device__ __forceinline__ uint32_t bf16_round(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;  // quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;                                // nearest even
}

// Accumulator for the elements of one 4-byte payload word.
template <int DT> struct Word;

template <> struct Word<DT_F32> {
  float a;
  __device__ __forceinline__ static Word widen(uint32_t w) { return {__uint_as_float(w)}; }
  __device__ __forceinline__ void add(const Word& o) { a = a + o.a; }
  __device__ __forceinline__ uint32_t narrow() const { return __float_as_uint(a); }
};

template <> struct Word<DT_I32> {
  uint32_t a;
  __device__ __forceinline__ static Word widen(uint32_t w) { return {w}; }
  __device__ __forceinline__ void add(const Word& o) { a = a + o.a; }  // wraps
  __device__ __forceinline__ uint32_t narrow() const { return a; }
};

template <> struct Word<DT_BF16> {
  float lo, hi;  // element 0 in the low half-word, element 1 in the high one
  __device__ __forceinline__ static Word widen(uint32_t w) {
    return {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  }
  __device__ __forceinline__ void add(const Word& o) { lo = lo + o.lo; hi = hi + o.hi; }
  __device__ __forceinline__ uint32_t narrow() const { return bf16_round(lo) | (bf16_round(hi) << 16); }
};

// A 16-byte vector of payload as four word accumulators.
template <int DT> struct Vec {
  Word<DT> w[4];
  __device__ __forceinline__ static Vec widen(const uint4& v) {
    Vec r;
    r.w[0] = Word<DT>::widen(v.x); r.w[1] = Word<DT>::widen(v.y);
    r.w[2] = Word<DT>::widen(v.z); r.w[3] = Word<DT>::widen(v.w);
    return r;
  }
  __device__ __forceinline__ void add(const Vec& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i].add(o.w[i]);
  }
  __device__ __forceinline__ uint4 narrow() const {
    return make_uint4(w[0].narrow(), w[1].narrow(), w[2].narrow(), w[3].narrow());
  }
};

// One payload element (tails and unaligned slices), as an accumulator.
template <int DT> struct Elem {
  static constexpr int size = (DT == DT_BF16) ? 2 : 4;
  __device__ __forceinline__ static float ldf(const char* p) {
    if (DT == DT_BF16) return __uint_as_float((uint32_t)(*(const uint16_t*)p) << 16);
    return *(const float*)p;
  }
  __device__ __forceinline__ static void stf(char* p, float v) {
    if (DT == DT_BF16) *(uint16_t*)p = (uint16_t)bf16_round(v);
    else *(float*)p = v;
  }
};

// ------------------------------------------------------------ memory access
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const char* p) { return *(const uint4*)p; }
__device__ __forceinline__ void st16(char* p, const uint4& v) { *(uint4*)p = v; }
// Streaming accesses: data read or written once per call is marked
// non-temporal, so it does not displace data that a later step re-reads
// (measured: +3% on the ring and two-shot, while one-shot, whose N rank
// programs re-read the same inputs, must keep its loads cached).
template <bool NT>
__device__ __forceinline__ uint4 ld16_hint(const char* p) {
  if (NT) {
    const v4u32 v = __builtin_nontemporal_load((const v4u32*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  return ld16(p);
}
template <bool NT>
__device__ __forceinline__ void st16_hint(char* p, const uint4& x) {
  if (NT) {
    const v4u32 v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, (v4u32*)p);
  } else {
    st16(p, x);
  }
}

// Load a 16-byte vector of which only `nbytes` (< 16, whole elements) exist;
// the rest reads as zero.  `esize` = 2 or 4.  Fixed-trip unrolled loops keep
// every index a constant, so the vector stays in registers.
__device__ __forceinline__ uint4 ld_partial(const char* p, uint32_t nbytes, int esize) {
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int b = 0; b < 16; b += 2) {
    if ((uint32_t)b < nbytes && (esize == 2 || (b & 3) == 0)) {
      const uint32_t v = (esize == 2) ? (uint32_t)(*(const uint16_t*)(p + b)) : *(const uint32_t*)(p + b);
      w[b >> 2] |= v << ((b & 3) * 8);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void st_partial(char* p, const uint4& v, uint32_t nbytes, int esize) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int b = 0; b < 16; b += 2) {
    if ((uint32_t)b < nbytes && (esize == 2 || (b & 3) == 0)) {
      const uint32_t x = w[b >> 2] >> ((b & 3) * 8);
      if (esize == 2) *(uint16_t*)(p + b) = (uint16_t)x;
      else *(uint32_t*)(p + b) = x;
    }
  }
}

// Load / store `nbytes` (<= 16, whole elements) at a pointer that may be only
// element-aligned.
__device__ __forceinline__ uint4 ld_any(const char* p, uint32_t nbytes, int esize) {
  if (nbytes == 16 && ((uintptr_t)p & 15) == 0) return ld16(p);
  return ld_partial(p, nbytes, esize);
}
__device__ __forceinline__ void st_any(char* p, const uint4& v, uint32_t nbytes, int esize) {
  if (nbytes == 16 && ((uintptr_t)p & 15) == 0) st16(p, v);
  else st_partial(p, v, nbytes, esize);
}

// ------------------------------------------------------------------ atomics
__device__ __forceinline__ uint64_t ld_flag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Raise a flag to v: flag values only grow within and across calls, so an
// atomic max can never move a flag backwards, whatever the order in which
// signals land.
__device__ __forceinline__ void raise_flag(uint64_t* p, uint64_t v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this wave issued has completed.  For a
// device-scope (sc1) store, completion means it is visible device-wide.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------- device-coherent data accesses
// Data one rank program writes and another reads within the same call moves
// through device-scope accesses (cache policy sc1): stores write through the
// writer's XCD L2 and complete only once visible device-wide; loads return
// device-coherent data.  A producer's data stores therefore complete before
// its flag store is issued (wait_mem), and a consumer's data loads are issued
// after it has seen the flag.  This replaces agent-scope release fences,
// whose L2 write-back of the whole XCD cache measured 3-7x slower per 64 KiB
// tile than plain streaming, while sc1 streaming runs at plain speed.
constexpr int CPOL_SC1 = 16;             // buffer-instruction cache policy: device scope
constexpr int RSRC_WORD3 = 0x00020000;   // raw buffer, 32-bit data format (CDNA)

typedef __amdgpu_buffer_rsrc_t Rsrc;

// A buffer resource over [base, base + bytes); offsets are 32-bit, so one is
// made per tile.  Out-of-range accesses are dropped by the hardware.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, RSRC_WORD3);
}
__device__ __forceinline__ uint4 cld16(Rsrc r, uint32_t off) {
  const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_SC1);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void cst16(Rsrc r, uint32_t off, const uint4& x) {
  const v4u32 v = {x.x, x.y, x.z, x.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CPOL_SC1);
}
__device__ __forceinline__ uint2 cld8(Rsrc r, uint32_t off) {
  typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
  const v2u32 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CPOL_SC1);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void cst8(Rsrc r, uint32_t off, const uint2& x) {
  typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
  const v2u32 v = {x.x, x.y};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CPOL_SC1);
}
// `nbytes` (< 16, whole elements of `esize` bytes) at offset `off`; zero-filled.
__device__ __forceinline__ uint4 cld_partial(Rsrc r, uint32_t off, uint32_t nbytes, int esize) {
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int b = 0; b < 16; b += 2) {
    if ((uint32_t)b < nbytes && (esize == 2 || (b & 3) == 0)) {
      const uint32_t v = (esize == 2)
          ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off + b, 0, CPOL_SC1)
          : __builtin_amdgcn_raw_buffer_load_b32(r, off + b, 0, CPOL_SC1);
      w[b >> 2] |= v << ((b & 3) * 8);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void cst_partial(Rsrc r, uint32_t off, const uint4& x, uint32_t nbytes, int esize) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int b = 0; b < 16; b += 2) {
    if ((uint32_t)b < nbytes && (esize == 2 || (b & 3) == 0)) {
      const uint32_t v = w[b >> 2] >> ((b & 3) * 8);
      if (esize == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, r, off + b, 0, CPOL_SC1);
      else __builtin_amdgcn_raw_buffer_store_b32(v, r, off + b, 0, CPOL_SC1);
    }
  }
}

// ---------------------------------------------------------- control block
// Lives at the start of the communicator's workspace (zeroed at creation).
// Each hot word on its own 128-byte line: the ticket counter is hammered by
// every workgroup, the abort word is polled, the epoch is read at start.
struct Ctl {
  uint32_t ticket;    // next task ticket of the running call
  uint32_t die_next[8];  // by-die calls: next ticket index of each die's share
  uint32_t pad0[23];
  uint32_t done;      // workgroups of the running call that have finished
  uint32_t pad1[31];
  uint64_t epoch;     // calls completed on this communicator
  uint64_t pad2[15];
  uint32_t abort;     // a wait timed out: every rank program gives up
  uint32_t err_code;  // 0 or the ar_status of the latched error
  uint32_t err_key;   // min over blocked waits of (step << 8 | rank), ~0 if none
  uint32_t pad3[29];
  // Diagnostics of the first wait that timed out: set, flag word index,
  // value seen, value awaited, call counter; then tasks finished this call.
  uint64_t diag[6];
  uint64_t pad4[10];
};

struct KArgs {
  const char* in[MAX_RANKS];
  char* out[MAX_RANKS];
  Geometry g;
  Ctl* ctl;
  uint64_t* flags;
  char* lines;          // LL / LL128 staging
  char* stage;          // ring reduce-scatter partials: one full buffer per rank
  uint64_t stage_stride;
  uint64_t timeout;     // wall-clock ticks (100 MHz) a wait may last
  int32_t inj_rank, inj_step;
  uint32_t batch;       // tickets a workgroup takes per fetch
  uint32_t fixed;       // 1: workgroup b runs tickets [b*batch, (b+1)*batch) and
                        //    touches no counter (tasks that never wait, one pass)
  uint32_t fold;        // 1: one-shot tasks load every term of a pass at once
  uint32_t rearm_errors;  // 1: the last workgroup out also clears the abort word
                          //    and error record (workspaces no host call resets)
  uint32_t colocate;      // 1: launched as a colocated kernel, workgroup b = (tile b/N, rank b%N)
  uint32_t by_die;        // G > 0: each run of G tickets sharing a tile runs on one die (die_ticket;
                          //        ticketed calls fetch from their die's counter, die_next)
};

__device__ __forceinline__ void note_blocked(Ctl* c, int step, int rank) {
  __hip_atomic_fetch_min(&c->err_key, (uint32_t)((step << 8) | rank), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void record_timeout(Ctl* c, const uint64_t* base, const uint64_t* f, uint64_t seen,
                                               uint64_t target) {
  if (__hip_atomic_fetch_add(&c->diag[0], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
    __hip_atomic_store(&c->diag[1], (uint64_t)(f - base), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->diag[2], seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->diag[3], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->diag[4], __hip_atomic_load(&c->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void raise_timeout(Ctl* c, int step, int rank) {
  note_blocked(c, step, rank);
  __hip_atomic_store(&c->err_code, 6u /* AR_ERR_TIMEOUT */, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&c->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every poll loop reads the shared abort word and the real-time clock only
// once per POLL_CHECK_EVERY polls.  Both are slow to read (the abort word is
// one address that every waiting wave shares; the clock is a scalar memory
// message): read at every poll, they made each step of a small ring cost
// 10-20 us.  A wait's time limit starts at its first check.
constexpr uint32_t POLL_CHECK_EVERY = 64;
enum PollState { POLL_GO = 0, POLL_ABORTED = 1, POLL_TIMED_OUT = 2 };

struct PollClock {
  uint32_t polls = 0;
  bool started = false;
  uint64_t t0 = 0;
  __device__ __forceinline__ int tick(const KArgs& a) {
    if (++polls % POLL_CHECK_EVERY) return POLL_GO;
    if (ld_u32(&a.ctl->abort)) return POLL_ABORTED;
    const uint64_t now = wall_clock64();
    if (!started) { started = true; t0 = now; return POLL_GO; }
    return (now - t0 > a.timeout) ? POLL_TIMED_OUT : POLL_GO;
  }
};

// Sleep before the next poll of a wait that is not yet satisfied: from ~50 ns
// doubling up to ~0.85 us (s_sleep counts 64 clocks per unit).  Every poll
// loop backs off: a line or flag being polled sits in the same memory channel
// as the producer's stores to it, and thousands of lanes re-polling at full
// rate would queue ahead of those stores and starve the producers.
__device__ __forceinline__ void poll_sleep(uint32_t& level) {
  for (uint32_t i = 0; i < (1u << level); ++i) __builtin_amdgcn_s_sleep(2);
  if (level < 4) ++level;
}

// Bounded spin of ONE thread until *f >= target.  Returns false if the call
// is aborted (by this wait timing out or by another one).
__device__ __forceinline__ bool wait_ge(const uint64_t* f, uint64_t target, const KArgs& a, int step,
                                        int rank) {
  if (ld_flag(f) >= target) return true;
  PollClock clock;
  uint32_t level = 0;
  while (true) {
    poll_sleep(level);
    if (ld_flag(f) >= target) return true;
    const int st = clock.tick(a);
    if (st == POLL_ABORTED) { note_blocked(a.ctl, step, rank); return false; }
    if (st == POLL_TIMED_OUT) {
      record_timeout(a.ctl, a.flags, f, ld_flag(f), target);
      raise_timeout(a.ctl, step, rank);
      return false;
    }
  }
}

}  // namespace ar
