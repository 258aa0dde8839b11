// kernels.hip -- gfx950 kernels of the all-reduce family.
//
// One persistent kernel per call.  Each workgroup (256 threads, 4 wave64s)
// repeatedly takes a ticket, decodes it into a task (schedule.hpp) and runs
// it: one rank program's work on one tile.  Payload moves through HBM in
// 16-byte vectors (global_load/store_dwordx4), several vectors in flight per
// thread.  This is a streaming reduction (under 0.1 flop per byte): no MFMA,
// the bound is HBM bandwidth.
//
// Which rank reads and writes what at each step follows "Collective
// communication: NCCL's algorithms and protocols, and custom all-reduce",
// section "Algorithms" (ring, one-shot, two-shot) and "NCCL collectives, ring
// all-reduce & launching TP/PP", section "Direct answer" (reduce-scatter,
// all-gather, ring = reduce-scatter + all-gather); the transfer encodings
// follow the former page's section "Protocols" (see device.hpp).
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "call.hpp"

namespace ar {

// Values every thread of a workgroup holds equal (read back from LDS), made
// visibly uniform to the compiler.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  return ((uint64_t)uniform((uint32_t)(x >> 32)) << 32) | uniform((uint32_t)x);
}

constexpr int U_SIMPLE = 4;  // 16-byte vectors in flight per thread per source
constexpr int U_LL = 4;      // LL words per thread per pass
constexpr int U_LL128 = 4;   // LL128 line groups (8 lines of a wave) per pass of the N-term gather
constexpr int U_LL128_PASS = 4;  // ... and per pass of a one- or two-term pass (ring, send, copy)

// =============================================================== Simple path
// dst = fold(term(0), ..., term(n-1)) over `nbytes` (whole elements, at most
// 64 KiB: one tile).  One term = raw copy (bit-exact for every type).
// COH_TERMS: bit i set = term(i) was written by another rank program during
// this call (read at device scope); a plain `true` marks term(0) only.
// COH_DST: dst will be read by another rank program during this call
// (written at device scope).  Other terms are inputs.
// NT_IN: inputs are read once per call; NT_OUT: a plain dst is final output.
template <int DT, unsigned COH_TERMS, bool COH_DST, bool NT_IN = true, bool NT_OUT = true, class Term>
__device__ __forceinline__ void simple_stream(Term term, int nterms, char* dst, uint64_t nbytes) {
  constexpr bool COH_FIRST = (COH_TERMS & 1u) != 0;
  const int es = Elem<DT>::size;
  const char* t0 = term(0);
  const Rsrc r0 = make_rsrc(t0, (uint32_t)nbytes);
  const Rsrc rd = make_rsrc(dst, (uint32_t)nbytes);
  bool aligned = (((uintptr_t)dst | (uintptr_t)t0) & 15) == 0;
  for (int i = 1; i < nterms; ++i) aligned = aligned && (((uintptr_t)term(i) & 15) == 0);
  const uint32_t nfull = aligned ? (uint32_t)(nbytes / 16) : 0u;
  for (uint32_t base = threadIdx.x; base < nfull; base += U_SIMPLE * WG_THREADS) {
    uint4 x[U_SIMPLE];
    Vec<DT> acc[U_SIMPLE];
#pragma unroll
    for (int u = 0; u < U_SIMPLE; ++u) {
      const uint32_t v = base + u * WG_THREADS;
      x[u] = make_uint4(0, 0, 0, 0);
      if (v < nfull) x[u] = COH_FIRST ? cld16(r0, v * 16) : ld16_hint<NT_IN>(t0 + (uint64_t)v * 16);
    }
    if (nterms == 1) {
#pragma unroll
      for (int u = 0; u < U_SIMPLE; ++u) {
        const uint32_t v = base + u * WG_THREADS;
        if (v < nfull) {
          if (COH_DST) cst16(rd, v * 16, x[u]);
          else st16_hint<NT_OUT>(dst + (uint64_t)v * 16, x[u]);
        }
      }
      continue;
    }
#pragma unroll
    for (int u = 0; u < U_SIMPLE; ++u) acc[u] = Vec<DT>::widen(x[u]);
    for (int i = 1; i < nterms; ++i) {
      const char* p = term(i);
      if ((COH_TERMS >> i) & 1u) {
        const Rsrc rp = make_rsrc(p, (uint32_t)nbytes);
#pragma unroll
        for (int u = 0; u < U_SIMPLE; ++u) {
          const uint32_t v = base + u * WG_THREADS;
          x[u] = (v < nfull) ? cld16(rp, v * 16) : make_uint4(0, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U_SIMPLE; ++u) {
          const uint32_t v = base + u * WG_THREADS;
          x[u] = (v < nfull) ? ld16_hint<NT_IN>(p + (uint64_t)v * 16) : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < U_SIMPLE; ++u) acc[u].add(Vec<DT>::widen(x[u]));
    }
#pragma unroll
    for (int u = 0; u < U_SIMPLE; ++u) {
      const uint32_t v = base + u * WG_THREADS;
      if (v < nfull) {
        if (COH_DST) cst16(rd, v * 16, acc[u].narrow());
        else st16_hint<NT_OUT>(dst + (uint64_t)v * 16, acc[u].narrow());
      }
    }
  }
  // Remainder (and every vector of a misaligned range): element-exact path.
  const uint32_t done = nfull * 16;
  const uint32_t nrest = (uint32_t)cdiv(nbytes - done, 16);
  for (uint32_t v = threadIdx.x; v < nrest; v += WG_THREADS) {
    const uint32_t off = done + v * 16;
    const uint32_t nb = (uint32_t)umin(16, nbytes - off);
    uint4 x = COH_FIRST ? cld_partial(r0, off, nb, es) : ld_any(t0 + off, nb, es);
    if (nterms > 1) {
      Vec<DT> acc = Vec<DT>::widen(x);
      for (int i = 1; i < nterms; ++i) {
        const uint4 y = ((COH_TERMS >> i) & 1u) ? cld_partial(make_rsrc(term(i), (uint32_t)nbytes), off, nb, es)
                                                 : ld_any(term(i) + off, nb, es);
        acc.add(Vec<DT>::widen(y));
      }
      x = acc.narrow();
    }
    if (COH_DST) cst_partial(rd, off, x, nb, es);
    else st_any(dst + off, x, nb, es);
  }
}

// Raw-buffer 16-byte accesses with a non-temporal hint (cache policy nt):
// the buffer forms let one pass load every term with no per-lane bounds
// branch (an access past the resource's end reads zeros, a store there is
// dropped), and a scheduling barrier then keeps every load in flight before
// the first add.
constexpr int CPOL_NT = 2;
template <bool NT>
__device__ __forceinline__ uint4 bld16(Rsrc r, uint32_t off) {
  const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? CPOL_NT : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <bool NT>
__device__ __forceinline__ void bst16(Rsrc r, uint32_t off, const uint4& x) {
  const v4u32 v = {x.x, x.y, x.z, x.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, NT ? CPOL_NT : 0);
}

// Vectors per thread per term of a fold pass, for about VECS loads in flight
// per thread whatever the term count (at most 8 per term).  Loading one term
// after another keeps only 4 vectors per thread in flight; with ~768 resident
// workgroups that is about 12 MiB GPU-wide, too little to cover HBM latency
// under load.  Measured at N=8, 256 MiB fp32: the two-shot (fold tasks
// interleaved with the gather tasks) runs 852 us with one term at a time, 824
// with 16 loads in flight and 791 with 32.  More in flight costs registers:
// the one-shot kernel with 32 needs 173 VGPRs, which leaves room for only two
// workgroups per CU, so its fold keeps 16.
template <int NTERMS, int VECS>
constexpr int fold_unroll() {
  return VECS / NTERMS >= 8 ? 8 : (VECS / NTERMS >= 1 ? VECS / NTERMS : 1);
}

// One payload element at byte offset `off` of a buffer resource, as a word
// whose low element is the payload (bf16 in the low half-word).
template <int DT>
__device__ __forceinline__ uint32_t bld_elem(Rsrc r, uint32_t off) {
  if constexpr (DT == DT_BF16) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// dst = term(0) + term(1) + ... + term(NTERMS-1), element by element in
// that order, over `nbytes` of one tile, for terms that are all inputs of the
// call (ready at launch: the one-shot and the two-shot's reduce half).
// Every term's vectors of a pass are loaded before the first add.  The tail
// of a block, and every element of a range that is not 16-byte aligned (the
// all-reduce blocks always are; the check keeps the fold safe for any
// caller), take one element per thread through the same buffer resources.
// NT_IN: inputs are read once per call; NT_OUT: dst is final output;
// COH_DST: dst is read by another rank program during this call.
template <int DT, int NTERMS, int VECS, bool NT_IN, bool NT_OUT, bool COH_DST, class Term>
__device__ __forceinline__ void fold_inputs(Term term, char* dst, uint64_t nbytes) {
  constexpr int UF = fold_unroll<NTERMS, VECS>();
  constexpr uint32_t ES = Elem<DT>::size;
  bool aligned = ((uintptr_t)dst & 15) == 0;
#pragma unroll
  for (int i = 0; i < NTERMS; ++i) aligned = aligned && (((uintptr_t)term(i) & 15) == 0);
  const uint32_t nfull = aligned ? (uint32_t)(nbytes / 16) : 0u;
  Rsrc rt[NTERMS];
#pragma unroll
  for (int i = 0; i < NTERMS; ++i) rt[i] = make_rsrc(term(i), (uint32_t)nbytes);
  const Rsrc rd = make_rsrc(dst, (uint32_t)nbytes);
  for (uint32_t base = threadIdx.x; base < nfull; base += UF * WG_THREADS) {
    // Group u of this pass starts at vector pass0 + u*WG_THREADS (the same
    // for the whole workgroup): groups wholly past the tile are skipped, so
    // a short tile does no work for the vectors it does not have.
    const uint32_t pass0 = uniform(base - threadIdx.x);
    uint4 x[UF][NTERMS];
#pragma unroll
    for (int u = 0; u < UF; ++u) {
      if (pass0 + u * WG_THREADS >= nfull) break;
#pragma unroll
      for (int i = 0; i < NTERMS; ++i) {
        // vectors past the last whole one read as zeros and are not stored
        const uint32_t v = base + u * WG_THREADS;
        x[u][i] = bld16<NT_IN>(rt[i], v < nfull ? v * 16 : 0xfffffff0u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UF; ++u) {
      if (pass0 + u * WG_THREADS >= nfull) break;
      Vec<DT> acc = Vec<DT>::widen(x[u][0]);
#pragma unroll
      for (int i = 1; i < NTERMS; ++i) acc.add(Vec<DT>::widen(x[u][i]));
      const uint32_t v = base + u * WG_THREADS;
      const uint32_t off = v < nfull ? v * 16 : 0xfffffff0u;
      if (COH_DST) cst16(rd, off, acc.narrow());
      else bst16<NT_OUT>(rd, off, acc.narrow());
    }
  }
  const uint32_t done = nfull * 16;
  const uint32_t nelem = ((uint32_t)nbytes - done) / ES;
  for (uint32_t e = threadIdx.x; e < nelem; e += WG_THREADS) {
    const uint32_t off = done + e * ES;
    Word<DT> acc = Word<DT>::widen(bld_elem<DT>(rt[0], off));
#pragma unroll
    for (int i = 1; i < NTERMS; ++i) acc.add(Word<DT>::widen(bld_elem<DT>(rt[i], off)));
    const uint32_t w = acc.narrow();
    if constexpr (DT == DT_BF16) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w, rd, off, 0, COH_DST ? CPOL_SC1 : 0);
    else __builtin_amdgcn_raw_buffer_store_b32(w, rd, off, 0, COH_DST ? CPOL_SC1 : 0);
  }
}

// fold_inputs over n terms (2..MAX_RANKS), n uniform.
template <int DT, int VECS, bool NT_IN, bool NT_OUT, bool COH_DST, class Term>
__device__ __forceinline__ void fold_n(Term term, int n, char* dst, uint64_t nbytes) {
  switch (n) {
    case 2: fold_inputs<DT, 2, VECS, NT_IN, NT_OUT, COH_DST>(term, dst, nbytes); break;
    case 3: fold_inputs<DT, 3, VECS, NT_IN, NT_OUT, COH_DST>(term, dst, nbytes); break;
    case 4: fold_inputs<DT, 4, VECS, NT_IN, NT_OUT, COH_DST>(term, dst, nbytes); break;
    case 5: fold_inputs<DT, 5, VECS, NT_IN, NT_OUT, COH_DST>(term, dst, nbytes); break;
    case 6: fold_inputs<DT, 6, VECS, NT_IN, NT_OUT, COH_DST>(term, dst, nbytes); break;
    case 7: fold_inputs<DT, 7, VECS, NT_IN, NT_OUT, COH_DST>(term, dst, nbytes); break;
    case 8: fold_inputs<DT, 8, VECS, NT_IN, NT_OUT, COH_DST>(term, dst, nbytes); break;
    default: simple_stream<DT, 0u, COH_DST, NT_IN, NT_OUT>(term, n, dst, nbytes); break;
  }
}

// simple_stream with the coherence choices made at run time (uniform values).
template <int DT, class Term>
__device__ __forceinline__ void stream(bool coh_first, bool coh_dst, Term term, int nterms, char* dst,
                                       uint64_t nbytes) {
  if (coh_first) {
    if (coh_dst) simple_stream<DT, true, true>(term, nterms, dst, nbytes);
    else simple_stream<DT, true, false>(term, nterms, dst, nbytes);
  } else {
    if (coh_dst) simple_stream<DT, false, true>(term, nterms, dst, nbytes);
    else simple_stream<DT, false, false>(term, nterms, dst, nbytes);
  }
}

// Workgroup waits until *f >= target (thread 0 polls with back-off); false
// if the call is aborted.  Thread 0's verdict is broadcast, so all waves take
// the same path through the barriers that follow.  The data the flag guards
// is read afterwards with device-scope (sc1) loads, issued only once thread
// 0's flag load has returned, so no acquire fence is needed: an agent-scope
// acquire would invalidate the XCD's whole L2 on every task (measured: 3% of
// ring bandwidth) and drop lines other tasks are about to reuse.
__device__ __forceinline__ bool wg_wait(const KArgs& a, const uint64_t* f, uint64_t target, int step,
                                        int rank) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    const bool ok = wait_ge(f, target, a, step, rank);
    s_ok = ok ? 1 : 0;
  }
  __syncthreads();
  // readfirstlane: the outcome is the same for the whole workgroup, and the
  // compiler must know it, or it may split the surrounding loop by lane.
  const bool ok = uniform(s_ok) != 0;
  __syncthreads();  // s_ok may be rewritten by the next wait
  return ok;
}

// Workgroup raises *f to v once every access of its task has completed: the
// device-scope data stores are then visible device-wide (and, for a
// read-done signal, every load has returned).  Exactly one lane signals: if
// every wave stored the flag, a late wave's store of step s could land after
// the next step's store of s+1 and move the flag backwards.  The barrier that
// ends every task in the ticket loop keeps this lane-0 store from sharing a
// divergent path with the next ticket fetch.
// The host's debug injection: rank program `rank` withholds what it sends at
// step `step` (a Simple signal, the flag of each LL or LL128 line).
__device__ __forceinline__ bool withheld(const KArgs& a, int step, int rank) {
  return rank == a.inj_rank && step == a.inj_step;
}

__device__ __forceinline__ void wg_signal(const KArgs& a, uint64_t* f, uint64_t v, int step, int rank) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0 && !withheld(a, step, rank)) raise_flag(f, v);
}

// ============================================================ LL / LL128 path
// A term of a line-processing pass: a plain buffer or a staging slot.
struct LTerm {
  const char* plain;  // payload bytes of the tile, or nullptr
  const char* lines;  // first line of the tile in staging, or nullptr
};

__device__ __forceinline__ uint32_t ld_word(const char* p, uint32_t nb, int es) {
  if (nb == 4 && ((uintptr_t)p & 3) == 0) return *(const uint32_t*)p;
  uint32_t w = 0;  // es == 2 here: one or two 2-byte elements
  if (nb > 0) w = *(const uint16_t*)p;
  if (nb > 2) w |= (uint32_t)(*(const uint16_t*)(p + 2)) << 16;
  return w;
}
__device__ __forceinline__ void st_word(char* p, uint32_t w, uint32_t nb, int es) {
  if (nb == 4 && ((uintptr_t)p & 3) == 0) { *(uint32_t*)p = w; return; }
  if (nb > 0) *(uint16_t*)p = (uint16_t)w;
  if (nb > 2) *(uint16_t*)(p + 2) = (uint16_t)(w >> 16);
}

// The first term of a pass that is a plain buffer (at most one per pass in
// every schedule: the rank's own input), or -1.  Its loads need no flag, so
// they go out with the first flag loads instead of a round trip later.
template <class Terms>
__device__ __forceinline__ int plain_term(Terms terms, int nterms) {
  for (int i = 0; i < nterms; ++i)
    if (terms(i).plain) return i;
  return -1;
}
// The first term that is a staging slot, or -1.
template <class Terms>
__device__ __forceinline__ int line_term(Terms terms, int nterms) {
  for (int i = 0; i < nterms; ++i)
    if (!terms(i).plain) return i;
  return -1;
}

// LL: 8-byte lines {payload word, flag}, written and read as one 64-bit
// agent-scope atomic.  Thread t handles words t, t+256, ... of the tile, so
// each wave's line stores and loads are contiguous.  A pass issues all its
// loads at once -- the plain term's words and the lines of every line term
// (one-shot and direct reduce-scatter receive N-1 of them) -- then checks
// the terms in order and re-polls only lines not yet written; the sum still
// runs in term order.
//
//   out_plain: store the result word here (may be null)
//   out_lines: put the result on the wire as lines (may be null)
template <int DT, class Terms>
__device__ __forceinline__ void ll_pass(const KArgs& a, Terms terms, int nterms, char* out_plain,
                                        char* out_lines, uint64_t nbytes, uint32_t flag, int step,
                                        int rank) {
  const int es = Elem<DT>::size;
  const uint64_t nwords = cdiv(nbytes, 4);
  const int pi = plain_term(terms, nterms);
  for (uint64_t base = threadIdx.x; base < nwords; base += (uint64_t)U_LL * WG_THREADS) {
    uint32_t pre[U_LL];
    if (pi >= 0) {
      const char* src = terms(pi).plain;
      // A pass of whole words (every pass but a tile's last) loads with no
      // branch, so the loads go out together.
      const uint64_t pass_end = (base - threadIdx.x + (uint64_t)U_LL * WG_THREADS) * 4;
      if (((uintptr_t)src & 3) == 0 && pass_end <= nbytes) {
#pragma unroll
        for (int u = 0; u < U_LL; ++u) pre[u] = *(const uint32_t*)(src + 4 * (base + (uint64_t)u * WG_THREADS));
      } else {
#pragma unroll
        for (int u = 0; u < U_LL; ++u) {
          const uint64_t w = base + (uint64_t)u * WG_THREADS;
          pre[u] = (w < nwords) ? ld_word(src + 4 * w, (uint32_t)umin(4, nbytes - 4 * w), es) : 0u;
        }
      }
    }
    uint64_t got[MAX_RANKS][U_LL];
#pragma unroll
    for (int i = 0; i < MAX_RANKS; ++i) {
      if (i >= nterms) break;
      const LTerm tm = terms(i);
      if (tm.plain) continue;
      const uint64_t* ln = (const uint64_t*)tm.lines;
#pragma unroll
      for (int u = 0; u < U_LL; ++u) {
        const uint64_t w = base + (uint64_t)u * WG_THREADS;
        got[i][u] = (w < nwords) ? ld_flag(ln + w) : ((uint64_t)flag << 32);
      }
    }
    uint32_t val[U_LL];
    Word<DT> acc[U_LL];
#pragma unroll
    for (int i = 0; i < MAX_RANKS; ++i) {
      if (i >= nterms) break;
      const LTerm tm = terms(i);
      if (i == pi) {
#pragma unroll
        for (int u = 0; u < U_LL; ++u) val[u] = pre[u];
      } else if (tm.plain) {
#pragma unroll
        for (int u = 0; u < U_LL; ++u) {
          const uint64_t w = base + (uint64_t)u * WG_THREADS;
          val[u] = (w < nwords) ? ld_word(tm.plain + 4 * w, (uint32_t)umin(4, nbytes - 4 * w), es) : 0u;
        }
      } else {
        const uint64_t* ln = (const uint64_t*)tm.lines;
        bool ready = true;
#pragma unroll
        for (int u = 0; u < U_LL; ++u) ready = ready && (uint32_t)(got[i][u] >> 32) == flag;
        if (!ready) {
          PollClock clock;
          uint32_t level = 0;
          while (true) {
            poll_sleep(level);
            ready = true;
#pragma unroll
            for (int u = 0; u < U_LL; ++u) {
              const uint64_t w = base + (uint64_t)u * WG_THREADS;
              if ((uint32_t)(got[i][u] >> 32) != flag) got[i][u] = ld_flag(ln + w);
              ready = ready && (uint32_t)(got[i][u] >> 32) == flag;
            }
            if (ready) break;
            const int st = clock.tick(a);
            if (st == POLL_ABORTED) { note_blocked(a.ctl, step, rank); break; }
            if (st == POLL_TIMED_OUT) { raise_timeout(a.ctl, step, rank); break; }
          }
        }
#pragma unroll
        for (int u = 0; u < U_LL; ++u) val[u] = (uint32_t)got[i][u];
      }
      if (nterms > 1) {
#pragma unroll
        for (int u = 0; u < U_LL; ++u) {
          const Word<DT> x = Word<DT>::widen(val[u]);
          if (i == 0) acc[u] = x; else acc[u].add(x);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U_LL; ++u) {
      const uint64_t w = base + (uint64_t)u * WG_THREADS;
      if (w >= nwords) continue;
      const uint32_t r = (nterms > 1) ? acc[u].narrow() : val[u];
      if (out_plain) st_word(out_plain + 4 * w, r, (uint32_t)umin(4, nbytes - 4 * w), es);
      if (out_lines && !withheld(a, step, rank)) st_flag((uint64_t*)out_lines + w, ((uint64_t)flag << 32) | r);
    }
  }
}

// Bytes [off, off+nb) of a tile, nb <= 16, whole elements, from a pointer
// that is at least element-aligned; 8-byte aligned 8/16-byte pieces load
// as dwordx2.
__device__ __forceinline__ uint4 ld_piece(const char* p, uint32_t nb, int es) {
  if (((uintptr_t)p & 7) == 0) {
    if (nb == 16) {
      const uint2 lo = *(const uint2*)p, hi = *(const uint2*)(p + 8);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    if (nb == 8) {
      const uint2 lo = *(const uint2*)p;
      return make_uint4(lo.x, lo.y, 0, 0);
    }
  }
  return ld_partial(p, nb, es);
}
__device__ __forceinline__ void st_piece(char* p, const uint4& v, uint32_t nb, int es) {
  if (((uintptr_t)p & 7) == 0) {
    if (nb == 16) { *(uint2*)p = make_uint2(v.x, v.y); *(uint2*)(p + 8) = make_uint2(v.z, v.w); return; }
    if (nb == 8) { *(uint2*)p = make_uint2(v.x, v.y); return; }
  }
  st_partial(p, v, nb, es);
}

// LL128: 128-byte lines {120 payload bytes, 8-byte flag}.  Lane q (0..7) of
// an 8-lane group owns bytes [16q, 16q+16) of its line: lanes 0..6 carry 16
// payload bytes, lane 7 carries 8 payload bytes and the flag.  Line L of a
// tile carries payload bytes [120L, 120L+120).  This pass takes one or two
// terms -- at most one plain buffer and one staging slot: a send, a ring
// step, a copy -- and each wave handles U_LL128_PASS groups of 8 consecutive
// lines per pass (1 KiB per store instruction).
//
// One round trip brings the plain term's pieces and the line term's flags;
// once every flag is seen, one more brings the line term's payload, all
// groups at once.  Payload moves a whole line per instruction: a line's
// bytes land as one full-line write instead of three partial ones (measured
// at 256 MiB fp32, N=8 ring: 4.91 -> 3.30 ms, HBM writes 30.4 S -> 26.7 S
// against 22.9 S of payload).  Holding each pass's flag stores back until
// the wave's next wait was tried as well: no faster at 256 MiB and slower at
// 2-32 MiB, where consumers then wait longer for every line.
template <int DT, class Terms>
__device__ __forceinline__ void ll128_pass(const KArgs& a, Terms terms, int nterms, char* out_plain,
                                           char* out_lines, uint64_t nbytes, uint64_t flag, int step,
                                           int rank) {
  constexpr int U = U_LL128_PASS;
  const int es = Elem<DT>::size;
  const uint64_t nlines = cdiv(nbytes, LL128_DATA);
  const int wave = uniform((int)(threadIdx.x / 64)), lane = threadIdx.x % 64;
  const int q = lane % 8, grp = lane / 8;
  const uint32_t lane_cap = (q < 7) ? 16u : 8u;
  const int pi = plain_term(terms, nterms);
  const int li = line_term(terms, nterms);
  const char* src_plain = pi >= 0 ? terms(pi).plain : nullptr;
  const char* src_lines = li >= 0 ? terms(li).lines : nullptr;
  const Rsrc rin = make_rsrc(src_lines ? src_lines : a.lines, src_lines ? (uint32_t)(nlines * LL128_LINE) : 0u);
  for (uint64_t l0 = (uint64_t)wave * U * 8; l0 < nlines; l0 += 4ull * U * 8) {
    uint32_t nb[U];  // payload bytes this lane owns in each of its lines
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t line = (uint32_t)(l0 + (uint64_t)u * 8 + grp);
      const uint64_t off = (uint64_t)line * LL128_DATA + 16ull * q;
      nb[u] = (line < nlines && off < nbytes) ? (uint32_t)umin(lane_cap, nbytes - off) : 0u;
    }
    // Loads that wait on nothing: the plain term, and the line term's flags
    // (every lane polls its own line's flag word; past the last line, a
    // harmless word).
    // A pass of whole lines (every pass but a short tile's last) loads the
    // plain pieces as two 8-byte halves per lane with no branch; lane 7,
    // which owns 8 bytes, loads its half twice and drops the copy.
    const bool whole = src_plain && ((uintptr_t)src_plain & 7) == 0 &&
                       (l0 + (uint64_t)U * 8) * LL128_DATA <= nbytes;
    uint4 pre[U];
    uint2 plo[U], phi[U];
    if (whole) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const char* p = src_plain + (l0 + (uint64_t)u * 8 + grp) * LL128_DATA + 16ull * q;
        plo[u] = *(const uint2*)p;
        phi[u] = *(const uint2*)(q < 7 ? p + 8 : p);
      }
    } else if (src_plain) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t off = (l0 + (uint64_t)u * 8 + grp) * LL128_DATA + 16ull * q;
        pre[u] = nb[u] ? ld_piece(src_plain + off, nb[u], es) : make_uint4(0, 0, 0, 0);
      }
    }
    // The flag word of group u's line (past the last line: line 0's, which
    // this pass reads anyway; one shared word for every idle lane of the GPU
    // would queue them all in one memory channel).
    auto flag_at = [&](int u) -> const uint64_t* {
      const uint64_t line = l0 + (uint64_t)u * 8 + grp;
      return (const uint64_t*)(src_lines + (line >= nlines ? 0 : line * LL128_LINE) + LL128_DATA);
    };
    bool ready[U];
    uint64_t fv[U];
    if (src_lines) {
#pragma unroll
      for (int u = 0; u < U; ++u) fv[u] = ld_flag(flag_at(u));
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used
    if (whole) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        pre[u] = q < 7 ? make_uint4(plo[u].x, plo[u].y, phi[u].x, phi[u].y) : make_uint4(plo[u].x, plo[u].y, 0, 0);
    }
    if (src_lines) {
      bool all = true;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ready[u] = l0 + (uint64_t)u * 8 + grp >= nlines || fv[u] == flag;
        all = all && ready[u];
      }
      if (!all) {
        PollClock clock;
        uint32_t level = 0;
        while (true) {
          poll_sleep(level);
          all = true;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (!ready[u]) ready[u] = ld_flag(flag_at(u)) == flag;
            all = all && ready[u];
          }
          if (all) break;
          const int st = clock.tick(a);
          if (st == POLL_ABORTED) { note_blocked(a.ctl, step, rank); break; }
          if (st == POLL_TIMED_OUT) { raise_timeout(a.ctl, step, rank); break; }
        }
      }
    }
    // Flags seen: the payload of every group at device scope, whole lines,
    // no branch between the loads (past the last line: zeros, nothing read).
    uint4 val[U];
    if (src_lines) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        val[u] = cld16(rin, (uint32_t)((l0 + (uint64_t)u * 8 + grp) * LL128_LINE) + 16u * q);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Sum in term order (term 0, then term 1), one group at a time.
    const Rsrc rout = make_rsrc(out_lines ? out_lines : a.lines, out_lines ? (uint32_t)(nlines * LL128_LINE) : 0u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t line = l0 + (uint64_t)u * 8 + grp;
      const uint64_t off = line * LL128_DATA + 16ull * q;
      uint4 lv = make_uint4(0, 0, 0, 0);
      if (src_lines && nb[u]) lv = q < 7 ? val[u] : make_uint4(val[u].x, val[u].y, 0, 0);
      const uint4 x0 = pi == 0 ? pre[u] : lv;
      uint4 res = x0;
      if (nterms > 1) {
        const uint4 x1 = pi == 1 ? pre[u] : lv;
        Vec<DT> acc = Vec<DT>::widen(x0);
        acc.add(Vec<DT>::widen(x1));
        res = acc.narrow();
      }
      if (out_plain && nb[u]) st_piece(out_plain + off, res, nb[u], es);
      // Whole line, flag word still 0 (never a valid flag); a partial lane
      // stores zero padding.
      if (out_lines && line < nlines)
        cst16(rout, (uint32_t)(line * LL128_LINE) + 16u * q, q < 7 ? res : make_uint4(res.x, res.y, 0, 0));
    }
    if (out_lines) {
      // ... complete (visible device-wide), then the flags.
      wait_mem();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t line = l0 + (uint64_t)u * 8 + grp;
        if (q == 7 && line < nlines && !withheld(a, step, rank))
          st_flag((uint64_t*)(out_lines + line * LL128_LINE + LL128_DATA), flag);
      }
    }
  }
}

// LL128 receive of a pass over many terms (one-shot and direct
// reduce-scatter receive, the two-shot fold: the own input and N-1 peers'
// lines).  Checking one term after another costs two round trips per peer
// (flag, then payload).  Here the flags of every line term come first, in one
// round trip: lane L checks line l0 + L%32 of terms 2k + L/32 (k = 0..3), so
// the wave covers all (term, line) pairs of its 32 lines.  Once the whole
// wave has seen them, each line group's payload of every term is loaded in
// one round trip and summed in term order.
template <int DT, class Terms>
__device__ __forceinline__ void ll128_gather(const KArgs& a, Terms terms, int nterms, char* out_plain,
                                             char* out_lines, uint64_t nbytes, uint64_t flag, int step,
                                             int rank) {
  const int es = Elem<DT>::size;
  const uint64_t nlines = cdiv(nbytes, LL128_DATA);
  const int wave = uniform((int)(threadIdx.x / 64)), lane = threadIdx.x % 64;
  const int q = lane % 8, grp = lane / 8;
  const uint32_t lane_cap = (q < 7) ? 16u : 8u;
  constexpr int FLAG_LOADS = (MAX_RANKS * 32 + 63) / 64;
  const int pi = plain_term(terms, nterms);
  const int li = line_term(terms, nterms);
  for (uint64_t l0 = (uint64_t)wave * U_LL128 * 8; l0 < nlines; l0 += 4ull * U_LL128 * 8) {
    {
      // Terms 2k and 2k+1 are evaluated for the wave (uniform), each lane
      // picks its own; lanes with nothing to check load a harmless word (the
      // first line term's line 0 flag, read anyway), so all loads go out
      // back to back.
      const uint64_t fl = l0 + lane % 32;
      const uint64_t* idle = li >= 0 ? (const uint64_t*)(terms(li).lines + LL128_DATA) : &a.ctl->epoch;
      const uint64_t* fp[FLAG_LOADS];
      bool ready[FLAG_LOADS];
#pragma unroll
      for (int k = 0; k < FLAG_LOADS; ++k) {
        const LTerm t0 = 2 * k < nterms ? terms(2 * k) : LTerm{nullptr, nullptr};
        const LTerm t1 = 2 * k + 1 < nterms ? terms(2 * k + 1) : LTerm{nullptr, nullptr};
        const char* ln = lane < 32 ? t0.lines : t1.lines;
        const bool check = ln != nullptr && fl < nlines;
        ready[k] = !check;
        fp[k] = check ? (const uint64_t*)(ln + fl * LL128_LINE + LL128_DATA) : idle;
      }
      uint64_t fv[FLAG_LOADS];
#pragma unroll
      for (int k = 0; k < FLAG_LOADS; ++k) fv[k] = ld_flag(fp[k]);
      bool all = true;
#pragma unroll
      for (int k = 0; k < FLAG_LOADS; ++k) {
        ready[k] = ready[k] || fv[k] == flag;
        all = all && ready[k];
      }
      if (!all) {
        PollClock clock;
        uint32_t level = 0;
        while (true) {
          poll_sleep(level);
          all = true;
#pragma unroll
          for (int k = 0; k < FLAG_LOADS; ++k) {
            if (!ready[k]) ready[k] = ld_flag(fp[k]) == flag;
            all = all && ready[k];
          }
          if (all) break;
          const int st = clock.tick(a);
          if (st == POLL_ABORTED) { note_blocked(a.ctl, step, rank); break; }
          if (st == POLL_TIMED_OUT) { raise_timeout(a.ctl, step, rank); break; }
        }
      }
    }
    // Every lane of the wave is past its polls: all flags of the pass are
    // seen.  Per line group, every term's piece in one round trip.
#pragma unroll
    for (int u = 0; u < U_LL128; ++u) {
      const uint32_t line = (uint32_t)(l0 + (uint64_t)u * 8 + grp);
      const uint64_t off = (uint64_t)line * LL128_DATA + 16ull * q;
      const uint32_t nb = (line < nlines && off < nbytes) ? (uint32_t)umin(lane_cap, nbytes - off) : 0u;
      // Every line term's piece with no branch between the loads, then the
      // plain term's piece, so they all go out before the first wait (a lane
      // past the tile's last line reads outside the buffer resource and gets
      // zeros; the plain term's slot reads through an empty one).
      uint4 x[MAX_RANKS];
      bool is_line[MAX_RANKS];
#pragma unroll
      for (int i = 0; i < MAX_RANKS; ++i) {  // no early exit: terms past nterms read nothing
        const LTerm tm = terms(i);             // address arithmetic only
        is_line[i] = i < nterms && tm.lines != nullptr;
        const Rsrc rl = make_rsrc(is_line[i] ? tm.lines : a.lines, is_line[i] ? (uint32_t)(nlines * LL128_LINE) : 0u);
        x[i] = cld16(rl, line * LL128_LINE + 16u * q);
      }
      uint4 xp = make_uint4(0, 0, 0, 0);
      if (pi >= 0 && nb) xp = ld_piece(terms(pi).plain + off, nb, es);
      // Nothing may use a loaded value before the last load is issued: the
      // scheduler would otherwise wait out each load before the next.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MAX_RANKS; ++i) {
        const uint4 lv = q < 7 ? x[i] : make_uint4(x[i].x, x[i].y, 0, 0);
        x[i] = !nb ? make_uint4(0, 0, 0, 0) : (is_line[i] ? lv : xp);
      }
      Vec<DT> acc = Vec<DT>::widen(x[0]);
#pragma unroll
      for (int i = 1; i < MAX_RANKS; ++i)
        if (i < nterms) acc.add(Vec<DT>::widen(x[i]));
      const uint4 res = nterms > 1 ? acc.narrow() : x[0];
      if (out_plain && nb) st_piece(out_plain + off, res, nb, es);
      if (out_lines && line < nlines) {
        const Rsrc rl = make_rsrc(out_lines, (uint32_t)(nlines * LL128_LINE));
        cst16(rl, line * LL128_LINE + 16u * q, q < 7 ? res : make_uint4(res.x, res.y, 0, 0));
      }
    }
    if (out_lines) {
      wait_mem();
#pragma unroll
      for (int u = 0; u < U_LL128; ++u) {
        const uint32_t line = (uint32_t)(l0 + (uint64_t)u * 8 + grp);
        if (q == 7 && line < nlines && !withheld(a, step, rank))
          st_flag((uint64_t*)(out_lines + (uint64_t)line * LL128_LINE + LL128_DATA), flag);
      }
    }
  }
}

// A line-protocol pass over many terms (see ll128_gather); LL's own pass
// already loads every term at once.
template <int DT, int PROTO, class Terms>
__device__ __forceinline__ void line_gather(const KArgs& a, Terms terms, int nterms, char* out_plain,
                                            char* out_lines, uint64_t nbytes, uint64_t epoch, int step,
                                            int rank) {
  if constexpr (PROTO == PROTO_LL) {
    const uint32_t flag = (uint32_t)(epoch % 0xffffffffull) + 1u;
    ll_pass<DT>(a, terms, nterms, out_plain, out_lines, nbytes, flag, step, rank);
  } else {
    ll128_gather<DT>(a, terms, nterms, out_plain, out_lines, nbytes, epoch + 1, step, rank);
  }
}

// One line-protocol pass, dispatched on the protocol.
template <int DT, int PROTO, class Terms>
__device__ __forceinline__ void line_pass(const KArgs& a, Terms terms, int nterms, char* out_plain,
                                          char* out_lines, uint64_t nbytes, uint64_t epoch, int step,
                                          int rank) {
  if constexpr (PROTO == PROTO_LL) {
    const uint32_t flag = (uint32_t)(epoch % 0xffffffffull) + 1u;
    ll_pass<DT>(a, terms, nterms, out_plain, out_lines, nbytes, flag, step, rank);
  } else {
    ll128_pass<DT>(a, terms, nterms, out_plain, out_lines, nbytes, epoch + 1, step, rank);
  }
}

// Staging address of tile `tile` of slot `slot`.
__device__ __forceinline__ char* slot_tile(const KArgs& a, uint64_t slot, uint64_t tile) {
  return a.lines + (slot * a.g.slot_lines + tile * a.g.tile_lines) * a.g.line_bytes;
}

// =================================================================== tasks
template <int DT, int PROTO, int KIND>
__device__ __forceinline__ void run_task(const KArgs& a, const Task& k, uint64_t epoch) {
  const Geometry& g = a.g;
  const int n = g.nranks;
  const uint64_t es = (uint64_t)g.esize;
  const uint64_t nbytes = (k.hi - k.lo) * es;
  const uint64_t tag = (epoch + 1) << 8;  // Simple flag values of this call

  if constexpr (KIND == K_COPY) {
    const uint64_t off = k.lo * es;
    simple_stream<DT, false, false>([&](int) { return a.in[0] + off; }, 1, a.out[0] + off, nbytes);
  }

  if constexpr (KIND == K_ONESHOT) {
    const uint64_t off = k.lo * es;
    const int r = k.rank;
    if constexpr (PROTO == PROTO_SIMPLE) {
      if (!g.in_place) {
        // every rank program of this tile re-reads the same inputs: keep them cached
        if (a.fold) fold_n<DT, 16, false, true, false>([&](int i) { return a.in[i] + off; }, n, a.out[r] + off, nbytes);
        else simple_stream<DT, false, false, false>([&](int i) { return a.in[i] + off; }, n, a.out[r] + off, nbytes);
        return;
      }
      // In place: every rank program of this tile reads all N inputs into
      // registers (a tile is at most 16 KiB: 4 vectors per thread), signals
      // that it has read (step 0), waits for the other N-1, then writes.
      const int es_i = (int)es;
      uint4 res[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t o = (threadIdx.x + (uint64_t)u * WG_THREADS) * 16;
        res[u] = make_uint4(0, 0, 0, 0);
        if (o < nbytes) {
          const uint32_t nb = (uint32_t)umin(16, nbytes - o);
          Vec<DT> acc = Vec<DT>::widen(ld_any(a.in[0] + off + o, nb, es_i));
          for (int i = 1; i < n; ++i) acc.add(Vec<DT>::widen(ld_any(a.in[i] + off + o, nb, es_i)));
          res[u] = acc.narrow();
        }
      }
      uint64_t* fl = a.flags + k.tile * n;
      wg_signal(a, fl + r, tag + 1, 0, r);
      bool ok = true;
      for (int i = 0; i < n && ok; ++i) ok = wg_wait(a, fl + i, tag + 1, 1, r);
      if (!ok) return;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t o = (threadIdx.x + (uint64_t)u * WG_THREADS) * 16;
        if (o < nbytes) st_any(a.out[r] + off + o, res[u], (uint32_t)umin(16, nbytes - o), es_i);
      }
    } else {
      if (k.phase == PH_SEND) {  // rank r puts its input tile on the wire once
        line_pass<DT, PROTO>(a, [&](int) { return LTerm{a.in[r] + off, nullptr}; }, 1, nullptr,
                             slot_tile(a, r, k.tile), nbytes, epoch, 0, r);
      } else {  // rank r sums all N in rank order: own input, peers' lines
        line_gather<DT, PROTO>(
            a,
            [&](int i) {
              if (i == r && !g.in_place) return LTerm{a.in[r] + off, nullptr};
              return LTerm{nullptr, slot_tile(a, i, k.tile)};
            },
            n, a.out[r] + off, nullptr, nbytes, epoch, 1, r);
      }
    }
  }

  if constexpr (KIND == K_TWOSHOT) {
    const uint64_t j = k.block;
    const uint64_t off = (block_lo(g, j) + k.lo) * es;
    const int r = k.rank;
    if constexpr (PROTO == PROTO_SIMPLE) {
      uint64_t* fl = a.flags + j * g.tiles + k.tile;
      if (k.phase == PH_FOLD) {  // shot 1: rank j sums block j of every rank
        // block j's sum is read back by the other ranks: device scope
        fold_n<DT, 32, true, true, true>([&](int i) { return a.in[i] + off; }, n, a.out[j] + off, nbytes);
        wg_signal(a, fl, tag + 1, 0, r);
      } else {  // shot 2: rank r reads block j's sum back
        if (!wg_wait(a, fl, tag + 1, 1, r)) return;
        simple_stream<DT, true, false>([&](int) { return (const char*)a.out[j] + off; }, 1, a.out[r] + off,
                                        nbytes);
      }
    } else {
      const uint64_t nn = (uint64_t)n * n;
      if (k.phase == PH_SEND) {  // rank r sends its slice of block j to owner j
        line_pass<DT, PROTO>(a, [&](int) { return LTerm{a.in[r] + off, nullptr}; }, 1, nullptr,
                             slot_tile(a, (uint64_t)r * n + j, k.tile), nbytes, epoch, 0, r);
      } else if (k.phase == PH_RECV_FOLD) {  // owner j sums, keeps and publishes block j
        line_gather<DT, PROTO>(
            a,
            [&](int i) {
              if ((uint64_t)i == j) return LTerm{a.in[j] + off, nullptr};
              return LTerm{nullptr, slot_tile(a, (uint64_t)i * n + j, k.tile)};
            },
            n, a.out[j] + off, slot_tile(a, nn + j, k.tile), nbytes, epoch, 1, r);
      } else {  // rank r receives block j's sum
        line_pass<DT, PROTO>(a, [&](int) { return LTerm{nullptr, slot_tile(a, nn + j, k.tile)}; }, 1,
                             a.out[r] + off, nullptr, nbytes, epoch, 2, r);
      }
    }
  }

  if constexpr (KIND == K_RS_DIRECT) {
    const uint64_t j = k.block;
    const uint64_t in_off = (block_lo(g, j) + k.lo) * es, out_off = k.lo * es;
    const int r = k.rank;
    if constexpr (PROTO == PROTO_SIMPLE) {
      // One term at a time, as for the ring: folding every term's loads at
      // once ran slower here at every depth and tile size tried (256 MiB:
      // 422 us against 430-490), and so did plain loads (447 us).  Plain
      // stores of the result measured 411 us against 422 non-temporal.
      simple_stream<DT, false, false, true, false>([&](int i) { return a.in[i] + in_off; }, n, a.out[j] + out_off,
                                                   nbytes);
    } else {
      if (k.phase == PH_SEND) {
        line_pass<DT, PROTO>(a, [&](int) { return LTerm{a.in[r] + in_off, nullptr}; }, 1, nullptr,
                             slot_tile(a, (uint64_t)r * n + j, k.tile), nbytes, epoch, 0, r);
      } else {
        line_gather<DT, PROTO>(
            a,
            [&](int i) {
              if ((uint64_t)i == j) return LTerm{a.in[j] + in_off, nullptr};
              return LTerm{nullptr, slot_tile(a, (uint64_t)i * n + j, k.tile)};
            },
            n, a.out[j] + out_off, nullptr, nbytes, epoch, 1, r);
      }
    }
  }

  if constexpr (KIND == K_AG_DIRECT) {
    const uint64_t j = k.block;
    const uint64_t in_off = k.lo * es, out_off = (block_lo(g, j) + k.lo) * es;
    const int r = k.rank;
    if constexpr (PROTO == PROTO_SIMPLE) {
      // shard j is read by every rank: keep it cached
      simple_stream<DT, false, false, false>([&](int) { return a.in[j] + in_off; }, 1, a.out[r] + out_off, nbytes);
    } else {
      if (k.phase == PH_SEND) {  // rank j publishes its shard and keeps its own copy
        line_pass<DT, PROTO>(a, [&](int) { return LTerm{a.in[j] + in_off, nullptr}; }, 1,
                             a.out[j] + out_off, slot_tile(a, j, k.tile), nbytes, epoch, 0, r);
      } else {
        line_pass<DT, PROTO>(a, [&](int) { return LTerm{nullptr, slot_tile(a, j, k.tile)}; }, 1,
                             a.out[r] + out_off, nullptr, nbytes, epoch, 1, r);
      }
    }
  }

  if constexpr (KIND == K_TREE) {
    // Half `tree` of the buffer on tree `tree`; this task is the node at heap
    // position p.  A node keeps its partial, and later the sum, in its own
    // output.  Flags per (tree, tile, position): tag+1 = partial ready,
    // tag+2 = sum ready (the root's up task, every other node's down task).
    const uint64_t tree = k.block;
    const int p = k.peer;
    const uint64_t off = (block_lo(g, tree) + k.lo) * es;
    uint64_t* fl = a.flags + (tree * g.tiles + k.tile) * (uint64_t)n;
    const int c1 = 2 * p + 1, c2 = 2 * p + 2;
    char* mine = a.out[k.rank] + off;
    if (k.phase == PH_TREE_UP) {
      if (c1 < n && !wg_wait(a, fl + c1, tag + 1, 0, k.rank)) return;
      if (c2 < n && !wg_wait(a, fl + c2, tag + 1, 0, k.rank)) return;
      const char* own = a.in[k.rank] + off;
      const char* left = c1 < n ? (const char*)a.out[tree_rank(n, tree, c1)] + off : nullptr;
      const char* right = c2 < n ? (const char*)a.out[tree_rank(n, tree, c2)] + off : nullptr;
      // own input, then the left and the right child's partial (device scope)
      auto terms = [&](int i) { return i == 0 ? own : (i == 1 ? left : right); };
      const int nt = 1 + (c1 < n) + (c2 < n);
      simple_stream<DT, 6u, true>(terms, nt, mine, nbytes);
      wg_signal(a, fl + p, tag + (p == 0 ? 2 : 1), 0, k.rank);
    } else {
      const int parent = (p - 1) / 2;
      if (!wg_wait(a, fl + parent, tag + 2, 1, k.rank)) return;
      const char* up = a.out[tree_rank(n, tree, parent)] + off;
      if (c1 < n) {  // this node's children copy the sum from here
        simple_stream<DT, 1u, true>([&](int) { return up; }, 1, mine, nbytes);
        wg_signal(a, fl + p, tag + 2, 1, k.rank);
      } else {
        simple_stream<DT, 1u, false>([&](int) { return up; }, 1, mine, nbytes);
      }
    }
  }

  if constexpr (KIND == K_RING) {
    const int j = (int)k.block;
    const int s = k.step, q = k.rank;
    const int steps = g.steps;
    const uint64_t boff = (block_lo(g, (uint64_t)j) + k.lo) * es;  // block coordinates
    const uint64_t loff = k.lo * es;                               // within a per-rank slice
    auto R = [&](int x) { return rank_mod((int64_t)x, n); };
    if constexpr (PROTO == PROTO_SIMPLE) {
      uint64_t* fl = a.flags + k.chain;
      if (s > 0 && !wg_wait(a, fl, tag + (uint64_t)s, s, q)) return;
      // A partial or copied block read by the next step's rank moves at
      // device scope; inputs and the last step's output do not.
      const bool last = (s == steps - 1);
      if (g.op == OP_ALLREDUCE) {
        if (s < n - 1) {  // reduce step: rank q adds its input to the partial from q-1
          const char* src = (s == 0) ? a.in[R(j + 1)] + boff : (const char*)a.out[R(j + 1 + s)] + boff;
          const char* own = a.in[q] + boff;
          stream<DT>(s > 0, true, [&](int i) { return i == 0 ? src : own; }, 2, a.out[q] + boff, nbytes);
        } else {          // copy step: rank q copies the finished block from q-1
          const char* src = a.out[R(q - 1)] + boff;
          stream<DT>(true, !last, [&](int) { return src; }, 1, a.out[q] + boff, nbytes);
        }
      } else if (g.op == OP_REDUCE_SCATTER) {
        const char* src = (s == 0) ? a.in[R(j + 1)] + boff
                                   : (const char*)(a.stage + (uint64_t)R(j + 1 + s) * a.stage_stride + boff);
        char* dst = (s == n - 2) ? a.out[j] + loff : a.stage + (uint64_t)q * a.stage_stride + boff;
        const char* own = a.in[q] + boff;
        stream<DT>(s > 0, !last, [&](int i) { return i == 0 ? src : own; }, 2, dst, nbytes);
      } else {  // all-gather: step 0 = rank j's own copy, step s = rank j+s receives
        const char* src = (s <= 1) ? a.in[j] + loff : (const char*)a.out[R(q - 1)] + boff;
        stream<DT>(s >= 2, s >= 1 && !last, [&](int) { return src; }, 1, a.out[q] + boff, nbytes);
      }
      if (s < steps - 1) wg_signal(a, fl, tag + (uint64_t)s + 1, s, q);
    } else {
      // Transfer x of block j (made by step x, read by step x+1) in slot
      // j*(steps-1)+x.
      auto wire = [&](int x) { return slot_tile(a, (uint64_t)j * (steps - 1) + x, k.tile); };
      const bool last = (s == steps - 1);
      if (g.op == OP_ALLREDUCE) {
        if (s == 0) {  // rank j+1 puts its block j on the wire
          line_pass<DT, PROTO>(a, [&](int) { return LTerm{a.in[q] + boff, nullptr}; }, 1, nullptr,
                               wire(0), nbytes, epoch, s, q);
        } else if (s <= n - 1) {  // reduce receive; rank j (s = n-1) keeps the sum
          const bool owner = (s == n - 1);
          line_pass<DT, PROTO>(
              a,
              [&](int i) { return i == 0 ? LTerm{nullptr, wire(s - 1)} : LTerm{a.in[q] + boff, nullptr}; },
              2, owner ? a.out[q] + boff : nullptr, wire(s), nbytes, epoch, s, q);
        } else {  // copy receive
          line_pass<DT, PROTO>(a, [&](int) { return LTerm{nullptr, wire(s - 1)}; }, 1, a.out[q] + boff,
                               last ? nullptr : wire(s), nbytes, epoch, s, q);
        }
      } else if (g.op == OP_REDUCE_SCATTER) {
        if (s == 0) {
          line_pass<DT, PROTO>(a, [&](int) { return LTerm{a.in[q] + boff, nullptr}; }, 1, nullptr,
                               wire(0), nbytes, epoch, s, q);
        } else {
          line_pass<DT, PROTO>(
              a,
              [&](int i) { return i == 0 ? LTerm{nullptr, wire(s - 1)} : LTerm{a.in[q] + boff, nullptr}; },
              2, last ? a.out[j] + loff : nullptr, last ? nullptr : wire(s), nbytes, epoch, s, q);
        }
      } else {
        if (s == 0) {  // rank j: own copy and first send
          line_pass<DT, PROTO>(a, [&](int) { return LTerm{a.in[j] + loff, nullptr}; }, 1, a.out[j] + boff,
                               wire(0), nbytes, epoch, s, q);
        } else {
          line_pass<DT, PROTO>(a, [&](int) { return LTerm{nullptr, wire(s - 1)}; }, 1, a.out[q] + boff,
                               last ? nullptr : wire(s), nbytes, epoch, s, q);
        }
      }
    }
  }
}

// ================================================================== kernel
// Kinds whose tasks never wait on another task: the copy, and with Simple
// the one-shot out of place and the direct reduce-scatter and all-gather
// (every input is ready when the kernel starts).
template <int PROTO, int KIND>
constexpr bool never_waits() {
  return KIND == K_COPY || (PROTO == PROTO_SIMPLE && (KIND == K_ONESHOT || KIND == K_RS_DIRECT || KIND == K_AG_DIRECT));
}

// A workgroup leaves the call (thread 0): counts its finished tasks, and the
// last workgroup out re-arms the counters and advances the call counter.
// Relaxed is enough: every ticket fetch and the epoch load of this workgroup
// have returned before this add is issued, and the next call's kernel starts
// after this one's end-of-kernel cache write-back.
__device__ __forceinline__ void finish_workgroup(const KArgs& a, uint32_t finished) {
  __hip_atomic_fetch_add(&a.ctl->diag[5], (uint64_t)finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t d = __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (d == gridDim.x - 1) {  // last workgroup out: rearm for the next call
    __hip_atomic_store(&a.ctl->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.by_die && !a.fixed)
      for (uint32_t x = 0; x < (uint32_t)XCDS; ++x)
        __hip_atomic_store(&a.ctl->die_next[x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&a.ctl->epoch, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.rearm_errors) {  // every other workgroup has exited: no wait can raise the abort again
      __hip_atomic_store(&a.ctl->abort, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctl->err_code, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctl->err_key, 0xffffffffu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctl->diag[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Workgroup 0 of a colocated call (thread 0) moves the call counter on.
// Every workgroup adds itself to `done` once its epoch load has returned, so a
// full count means no workgroup of the call can still read the old epoch.
// `counted` is a load of the count issued earlier, with the receive's loads.
// The wait ends in practice at once: a workgroup counts itself in before any
// wait of its own.  It is bounded all the same; it ignores the abort word,
// because a workgroup not yet counted in still reads the epoch after an abort.
__device__ __forceinline__ void advance_epoch(const KArgs& a, uint64_t epoch, uint32_t counted) {
  if (counted < gridDim.x) {
    uint32_t level = 0, polls = 0;
    uint64_t t0 = 0;
    while (true) {
      poll_sleep(level);
      if (ld_u32(&a.ctl->done) >= gridDim.x) break;
      if (++polls % POLL_CHECK_EVERY) continue;
      const uint64_t now = wall_clock64();
      if (!t0) t0 = now;
      else if (now - t0 > a.timeout) { raise_timeout(a.ctl, 0, 0); break; }
    }
  }
  __hip_atomic_store(&a.ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&a.ctl->epoch, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The send and the receive of a colocated LL (tile, rank), written out for
// latency: `pre` holds the rank's input words (the whole tile: `passes`
// passes of U_LL words per thread, loaded with the epoch).  They go on the
// wire as lines; then, pass by pass, every peer's lines load at once and the
// sum runs in rank order with `pre` as the rank's own term, as the generic
// pass sums it.  Bounded buffer accesses replace the per-lane tail
// branches: behind such a branch the compiler waited for each batch of
// loads before issuing the next (the generic pass took three round trips
// here, one for the input pointer, one for the input words, one for the
// lines).  While any line of a pass is missing, a poll reloads every peer
// line of the pass at once (a line already seen does not change during the
// call), so a late peer costs one round trip, not one per term; a reload of
// only the missing lines made the compiler wait after each term.
template <int DT, int PASSES>
__device__ __forceinline__ void colocated_ll(const KArgs& a, const Task& k, uint64_t epoch,
                                             const uint32_t (&pre)[PASSES][U_LL], int passes, uint64_t nbytes,
                                             uint32_t& counted) {
  const int n = a.g.nranks;
  const int r = k.rank;
  const uint32_t nwords = (uint32_t)cdiv(nbytes, 4);
  const uint32_t flag = (uint32_t)(epoch % 0xffffffffull) + 1u;
  // Staging of this tile for rank i: tile_lines + i * slot_stride (slot_tile,
  // computed once: per term, the compiler re-read the arguments and waited).
  const uint64_t slot_stride = uniform64(a.g.slot_lines * a.g.line_bytes);
  const char* tile_lines = a.lines + uniform64(k.tile * a.g.tile_lines * a.g.line_bytes);
  if (!withheld(a, 0, r)) {
    const Rsrc own = make_rsrc(tile_lines + (uint64_t)r * slot_stride, nwords * 8);
#pragma unroll
    for (int p = 0; p < PASSES; ++p)  // stores past the tile are dropped
#pragma unroll
      for (int u = 0; u < U_LL; ++u)
        cst8(own, 8 * (threadIdx.x + (uint32_t)(p * U_LL + u) * WG_THREADS), make_uint2(pre[p][u], flag));
  }
  // The peers store their lines at about the same time: loads issued before
  // this workgroup's own stores have landed mostly came back unwritten and
  // cost a poll (t=1 decode, N=8 bf16: 7.0 us per call without this wait,
  // 6.0 us with it).
  wait_mem();
  if (blockIdx.x == 0) counted = ld_u32(&a.ctl->done);
  const Rsrc out = make_rsrc(a.out[r] + k.lo * (uint64_t)Elem<DT>::size, (uint32_t)nbytes);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    if (p >= passes) break;
    const uint32_t base = threadIdx.x + (uint32_t)(p * U_LL) * WG_THREADS;  // word of u = 0
    uint2 got[MAX_RANKS][U_LL];  // (payload word, flag) of each peer's lines
#pragma unroll
    for (int i = 0; i < MAX_RANKS; ++i) {
      if (i >= n) break;
      if (i == r) continue;
      const Rsrc li = make_rsrc(tile_lines + (uint64_t)i * slot_stride, nwords * 8);
#pragma unroll
      for (int u = 0; u < U_LL; ++u) got[i][u] = cld8(li, 8 * (base + (uint32_t)u * WG_THREADS));
    }
    // Lanes past the tile read zeros and count as ready.
    auto missing = [&](int i, int u) { return base + (uint32_t)u * WG_THREADS < nwords && got[i][u].y != flag; };
    bool ready = true;
#pragma unroll
    for (int i = 0; i < MAX_RANKS; ++i) {
      if (i >= n) break;
      if (i == r) continue;
#pragma unroll
      for (int u = 0; u < U_LL; ++u) ready = ready && !missing(i, u);
    }
    if (!ready) {
      PollClock clock;
      uint32_t level = 0;
      while (true) {
        poll_sleep(level);
        ready = true;
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          if (i == r) continue;
          const Rsrc li = make_rsrc(tile_lines + (uint64_t)i * slot_stride, nwords * 8);
#pragma unroll
          for (int u = 0; u < U_LL; ++u) got[i][u] = cld8(li, 8 * (base + (uint32_t)u * WG_THREADS));
        }
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          if (i == r) continue;
#pragma unroll
          for (int u = 0; u < U_LL; ++u) ready = ready && !missing(i, u);
        }
        if (ready) break;
        const int st = clock.tick(a);
        if (st == POLL_ABORTED) { note_blocked(a.ctl, 1, r); return; }
        if (st == POLL_TIMED_OUT) { raise_timeout(a.ctl, 1, r); return; }
      }
    }
#pragma unroll
    for (int u = 0; u < U_LL; ++u) {
      uint32_t res = pre[p][u];
      if (n > 1) {
        Word<DT> acc;
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          const Word<DT> x = Word<DT>::widen(i == r ? pre[p][u] : got[i][u].x);
          if (i == 0) acc = x; else acc.add(x);
        }
        res = acc.narrow();
      }
      const uint32_t off = 4 * (base + (uint32_t)u * WG_THREADS);
      if constexpr (Elem<DT>::size == 2) {
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)res, out, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(res >> 16), out, off + 2, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(res, out, off, 0, 0);
      }
    }
  }
}

// LL128 counterpart of colocated_ll.  A workgroup pass is 128 lines: line
// L = 128 p + 32 wave + 8 u + group, lane q of the group owning bytes
// [16q, 16q+16) of it (lane 7: 8 payload bytes and the flag word).  `pre`
// holds the rank's payload pieces of every pass, loaded with the epoch.
// Send: every line whole with its flag word 0, wait until they are visible,
// then the flag words, and wait for those too (R15's order).  Receive, pass
// by pass: every peer's flag words at once (a poll reloads them all), then
// every peer's payload pieces at once, summed in rank order with `pre` as
// the rank's own term.  Bounded buffer accesses stand in for tail branches;
// per-element loads and stores keep ragged and 2-byte-aligned bf16 tails
// exact.
constexpr int U_C128 = 4;  // line groups of a wave per pass
// WORDS: every tile holds whole words (rank buffers are 16-byte aligned),
// so bf16 loads and stores go a word at a time too (the host checks).
template <int DT, bool WORDS = false>
__device__ __forceinline__ uint4 load_piece_bounded(Rsrc src, uint32_t off, bool full) {
  // `full`: 16 bytes (lanes 0..6), else 8 (lane 7); past the tile: zeros.
  const uint32_t hi = full ? off + 8 : 0x7ffffff0u;
  if constexpr (Elem<DT>::size == 2 && !WORDS) {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t o = (d < 2 ? off + 4 * d : hi + 4 * (d - 2));
      w[d] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src, o, 0, 0) |
             ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src, o + 2, 0, 0) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__builtin_amdgcn_raw_buffer_load_b32(src, off, 0, 0),
                      __builtin_amdgcn_raw_buffer_load_b32(src, off + 4, 0, 0),
                      __builtin_amdgcn_raw_buffer_load_b32(src, hi, 0, 0),
                      __builtin_amdgcn_raw_buffer_load_b32(src, hi + 4, 0, 0));
  }
}
template <int DT, bool WORDS = false>
__device__ __forceinline__ void store_piece_bounded(Rsrc dst, uint32_t off, bool full, const uint4& v) {
  const uint32_t hi = full ? off + 8 : 0x7ffffff0u;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t o = d < 2 ? off + 4 * d : hi + 4 * (d - 2);
    if constexpr (Elem<DT>::size == 2 && !WORDS) {
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w[d], dst, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[d] >> 16), dst, o + 2, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(w[d], dst, o, 0, 0);
    }
  }
}

template <int DT, int PASSES>
__device__ __forceinline__ void colocated_ll128(const KArgs& a, const Task& k, uint64_t epoch,
                                                const uint4 (&pre)[PASSES][U_C128], int passes, uint64_t nbytes,
                                                uint32_t& counted) {
  const int n = a.g.nranks;
  const int r = k.rank;
  const uint32_t nlines = (uint32_t)cdiv(nbytes, LL128_DATA);
  const uint64_t flag = epoch + 1;
  const uint32_t wave = uniform(threadIdx.x / 64), lane = threadIdx.x % 64, q = lane % 8, grp = lane / 8;
  const bool full = q < 7;
  auto line_of = [&](int p, int u) { return (uint32_t)(p * 128) + wave * 32 + (uint32_t)u * 8 + grp; };
  const uint64_t slot_stride = uniform64(a.g.slot_lines * a.g.line_bytes);
  const char* tile_lines = a.lines + uniform64(k.tile * a.g.tile_lines * a.g.line_bytes);
  const Rsrc own = make_rsrc(tile_lines + (uint64_t)r * slot_stride, nlines * LL128_LINE);
#pragma unroll
  for (int p = 0; p < PASSES; ++p)  // whole lines, flag word 0; past the tile: dropped
#pragma unroll
    for (int u = 0; u < U_C128; ++u)
      cst16(own, line_of(p, u) * LL128_LINE + 16 * q,
            full ? pre[p][u] : make_uint4(pre[p][u].x, pre[p][u].y, 0, 0));
  wait_mem();
  if (!withheld(a, 0, r)) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int u = 0; u < U_C128; ++u)  // lane 7 of each group: its line's flag word
        cst8(own, q == 7 ? line_of(p, u) * LL128_LINE + LL128_DATA : 0x7ffffff0u,
             make_uint2((uint32_t)flag, (uint32_t)(flag >> 32)));
  }
  wait_mem();
  if (blockIdx.x == 0) counted = ld_u32(&a.ctl->done);
  const Rsrc out = make_rsrc(a.out[r] + k.lo * (uint64_t)Elem<DT>::size, (uint32_t)nbytes);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    if (p >= passes) break;
    uint2 fl[MAX_RANKS][U_C128];
    auto load_flags = [&]() {
#pragma unroll
      for (int i = 0; i < MAX_RANKS; ++i) {
        if (i >= n) break;
        if (i == r) continue;
        const Rsrc li = make_rsrc(tile_lines + (uint64_t)i * slot_stride, nlines * LL128_LINE);
#pragma unroll
        for (int u = 0; u < U_C128; ++u) fl[i][u] = cld8(li, line_of(p, u) * LL128_LINE + LL128_DATA);
      }
    };
    auto all_seen = [&]() {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < MAX_RANKS; ++i) {
        if (i >= n) break;
        if (i == r) continue;
#pragma unroll
        for (int u = 0; u < U_C128; ++u)
          ok = ok && (line_of(p, u) >= nlines || (((uint64_t)fl[i][u].y << 32) | fl[i][u].x) == flag);
      }
      return ok;
    };
    load_flags();
    if (!all_seen()) {
      PollClock clock;
      uint32_t level = 0;
      while (true) {
        poll_sleep(level);
        load_flags();
        if (all_seen()) break;
        const int st = clock.tick(a);
        if (st == POLL_ABORTED) { note_blocked(a.ctl, 1, r); return; }
        if (st == POLL_TIMED_OUT) { raise_timeout(a.ctl, 1, r); return; }
      }
    }
    // Flags seen: the payload pieces, at device scope, all peers at once.
    uint4 pv[MAX_RANKS][U_C128];
#pragma unroll
    for (int i = 0; i < MAX_RANKS; ++i) {
      if (i >= n) break;
      if (i == r) continue;
      const Rsrc li = make_rsrc(tile_lines + (uint64_t)i * slot_stride, nlines * LL128_LINE);
#pragma unroll
      for (int u = 0; u < U_C128; ++u) pv[i][u] = cld16(li, line_of(p, u) * LL128_LINE + 16 * q);
    }
#pragma unroll
    for (int u = 0; u < U_C128; ++u) {
      uint4 res = pre[p][u];
      if (n > 1) {
        Vec<DT> acc;
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          const Vec<DT> x = Vec<DT>::widen(i == r ? pre[p][u] : pv[i][u]);
          if (i == 0) acc = x; else acc.add(x);
        }
        res = acc.narrow();
      }
      // Lane 7's upper half (the peers' flag words) is never stored.
      store_piece_bounded<DT>(out, line_of(p, u) * LL128_DATA + 16 * q, full, res);
    }
  }
}

// Small one-shot calls over LL / LL128 (g.colocated): workgroup b is rank
// b % N's program on tile b / N.  It puts its input tile on the wire, then
// gathers every rank's lines of the tile and sums them: the send and the
// receive of a (tile, rank) in one workgroup, with no ticket fetch between
// them.  The N workgroups of a tile wait on each other, so the grid (at most
// COLOCATED_WORKGROUPS) must be resident at once; launch_collective runs the
// ticketed schedule instead when the workgroup budget is smaller.
//
// Round trips of a decode-sized LL call: the epoch, loaded together with the
// rank's input words; the line stores; the loads of the peers' lines.  No
// workgroup waits on the return of an atomic: the last-workgroup-out count of
// the ticketed schedule is replaced by advance_epoch in workgroup 0.
template <int DT, int PROTO, int PASSES>
__device__ __forceinline__ void colocated_oneshot(const KArgs& a) {
  __shared__ uint64_t s_epoch;
  __shared__ uint32_t s_abort;
  const Geometry& g = a.g;
  const int n = g.nranks;
  Task k;
  // Scalar registers: a rank held in a vector register made the compiler
  // fetch a.in[rank] with a vector load and wait for it.
  k.rank = (int32_t)uniform(blockIdx.x % (uint32_t)n);
  k.peer = 0; k.step = 0; k.block = 0; k.chain = 0;
  k.tile = uniform(blockIdx.x / (uint32_t)n);
  tile_range(g, g.total, k.tile, &k.lo, &k.hi);
  const int r = k.rank;
  const int es = Elem<DT>::size;
  const uint64_t nbytes = (k.hi - k.lo) * (uint64_t)es;
  // Bounded buffer loads (bytes past the tile read as 0, with no memory
  // access) need no branch, per lane or per pass: behind a branch, the
  // compiler waited for these loads before the epoch load went out.  bf16
  // words load as two halves, since a bf16 tile may end mid-word (and a
  // half-covered word would read as zero).  The loads and stores of the
  // PASSES passes are all issued,
  // those past the tile included (they still cost address-unit time: a
  // one-pass tile in the 8-pass kernel took 2 us longer), hence a one-pass
  // kernel for one-pass tiles.
  uint32_t pre[PASSES][U_LL];
  uint4 pre128[PASSES][U_C128];
  int passes = 0;
  const Rsrc src = make_rsrc(a.in[r] + k.lo * (uint64_t)es, (uint32_t)nbytes);
  if constexpr (PROTO == PROTO_LL) {
    static_assert(U_LL * WG_THREADS * 4 == LL_COLOCATED_TILE, "a colocated LL pass is 4 KiB");
    passes = (int)cdiv(nbytes, LL_COLOCATED_TILE);  // at most PASSES (launch_collective)
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int u = 0; u < U_LL; ++u) {
        const uint32_t off = 4 * (threadIdx.x + (uint32_t)(p * U_LL + u) * WG_THREADS);
        if constexpr (Elem<DT>::size == 2)
          pre[p][u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src, off, 0, 0) |
                      ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src, off + 2, 0, 0) << 16);
        else
          pre[p][u] = __builtin_amdgcn_raw_buffer_load_b32(src, off, 0, 0);
      }
  } else {
    static_assert(4 * U_C128 * 8 * LL128_DATA == LL128_COLOCATED_PASS, "a colocated LL128 pass is 128 lines");
    passes = (int)cdiv(nbytes, LL128_COLOCATED_PASS);  // at most PASSES (launch_collective)
    const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int u = 0; u < U_C128; ++u) {
        const uint32_t line = (uint32_t)(p * 128) + wave * 32 + (uint32_t)u * 8 + lane / 8;
        pre128[p][u] = load_piece_bounded<DT>(src, line * LL128_DATA + 16 * (lane % 8), lane % 8 < 7);
      }
  }
  if (threadIdx.x == 0) {
    const uint64_t e = __hip_atomic_load(&a.ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ab = ld_u32(&a.ctl->abort);
    s_epoch = e;
    s_abort = ab;
  }
  __syncthreads();
  // Issued after the barrier, which follows the LDS store of the loaded
  // epoch: the count never runs ahead of the load.
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t epoch = uniform64(s_epoch);
  const bool aborted = uniform(s_abort) != 0;
  uint32_t finished = 0, counted = 0;
  if (!aborted && k.hi > k.lo) {  // a latched error: run nothing
    if constexpr (PROTO == PROTO_LL) {
      colocated_ll<DT, PASSES>(a, k, epoch, pre, passes, nbytes, counted);
    } else {
      colocated_ll128<DT, PASSES>(a, k, epoch, pre128, passes, nbytes, counted);
    }
    finished = 2;
  } else if (blockIdx.x == 0) {
    counted = ld_u32(&a.ctl->done);
  }
  // No barrier before the epoch moves on: it needs only the full count, and
  // behind a barrier (which waits for the output stores) workgroup 0's two
  // stores would land one round trip after every other workgroup's last.
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&a.ctl->diag[5], (uint64_t)finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0) advance_epoch(a, epoch, counted);
  }
}

// Loads one word of every 64-byte line of the kernel arguments, all issued
// before one wait, so the argument loads the compiler places later (each
// followed by a wait for its value) hit the scalar cache.  Without it a
// decode-sized call spent most of its time in such misses, one after another.
__device__ __forceinline__ void warm_kernel_args() {
  typedef const uint32_t __attribute__((address_space(4))) * KPtr;
  const KPtr p = (KPtr)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t x = 0;
#pragma unroll
  for (uint32_t i = 0; i < (sizeof(KArgs) + 63) / 64; ++i) x ^= p[16 * i];
  asm volatile("" ::"s"(x));
}

// Simple two-shots of mid-size blocks (a.colocate, make_geometry's rule):
// workgroup b is rank r = b % N on tile t = b / N of every block.  It folds
// tile t of its own block r over every rank's input (the ticketed fold:
// same summation order), raises that tile's flag (step 0), then, block by
// block starting after its own, waits for tile t's flag and copies the sum
// into its output (step 1).  The same flags, tags and steps as the ticketed
// schedule; in place is safe for the same reason: a block's sum is copied
// over a rank's input only after that block's owner has read it.
template <int DT>
__device__ __forceinline__ void colocated_twoshot_simple(const KArgs& a) {
  __shared__ uint64_t s_epoch;
  __shared__ uint32_t s_abort;
  const Geometry& g = a.g;
  const int n = g.nranks;
  const int r = (int)uniform(blockIdx.x % (uint32_t)n);
  const uint64_t t = uniform(blockIdx.x / (uint32_t)n);
  constexpr uint64_t es = Elem<DT>::size;
  if (threadIdx.x == 0) {
    const uint64_t e = __hip_atomic_load(&a.ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ab = ld_u32(&a.ctl->abort);
    s_epoch = e;
    s_abort = ab;
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t epoch = uniform64(s_epoch);
  const bool aborted = uniform(s_abort) != 0;
  const uint64_t tag = (epoch + 1) << 8;
  uint32_t finished = 0, counted = 0;
  if (!aborted) {
    uint64_t lo, hi;
    tile_range(g, block_len(g, (uint64_t)r), t, &lo, &hi);
    if (hi > lo) {
      const uint64_t off = (block_lo(g, (uint64_t)r) + lo) * es;
      fold_n<DT, 32, true, true, true>([&](int i) { return a.in[i] + off; }, n, a.out[r] + off, (hi - lo) * es);
      wg_signal(a, a.flags + (uint64_t)r * g.tiles + t, tag + 1, 0, r);
      ++finished;
    }
    if (blockIdx.x == 0) counted = ld_u32(&a.ctl->done);
    for (int k = 1; k < n; ++k) {
      const int j = (r + k) % n;
      tile_range(g, block_len(g, (uint64_t)j), t, &lo, &hi);
      if (hi <= lo) continue;
      if (!wg_wait(a, a.flags + (uint64_t)j * g.tiles + t, tag + 1, 1, r)) break;
      const uint64_t off = (block_lo(g, (uint64_t)j) + lo) * es;
      simple_stream<DT, true, false>([&](int) { return (const char*)a.out[j] + off; }, 1, a.out[r] + off,
                                      (hi - lo) * es);
      ++finished;
    }
  } else if (blockIdx.x == 0) {
    counted = ld_u32(&a.ctl->done);
  }
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&a.ctl->diag[5], (uint64_t)finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0) advance_epoch(a, epoch, counted);
  }
}

template <int DT>
__global__ __launch_bounds__(WG_THREADS) void colocated_twoshot_simple_kernel(KArgs a) {
  warm_kernel_args();
  colocated_twoshot_simple<DT>(a);
}

// Small LL128 two-shots (a.colocate): workgroup b is rank r = b % N on tile
// t = b / N of every block.  Step 0: r puts its tile t of every other block
// j on the wire to j (slot r*N + j).  Step 1: r gathers tile t of its own
// block from every peer (slot i*N + r), sums it in rank order with its own
// input, keeps it and publishes it (slot N*N + r).  Step 2: r copies tile t
// of every other block's sum (slot N*N + j) into its output.  Each step
// covers every pass of the tile before its one wait; the lines are those of
// colocated_ll128 (whole lines, flag word 0, then the flag words), the
// waits poll every line of a step at once.  In place is safe: a workgroup
// reads its input before writing the same bytes, and peers read only lines.
template <int DT, int PASSES, bool WORDS>
__device__ __forceinline__ void colocated_twoshot_ll128(const KArgs& a) {
  __shared__ uint64_t s_epoch;
  __shared__ uint32_t s_abort;
  const Geometry& g = a.g;
  const int n = g.nranks;
  const int r = (int)uniform(blockIdx.x % (uint32_t)n);
  const uint64_t t = uniform(blockIdx.x / (uint32_t)n);
  constexpr int es = Elem<DT>::size;
  const uint32_t wave = uniform(threadIdx.x / 64), lane = threadIdx.x % 64, q = lane % 8, grp = lane / 8;
  const bool full = q < 7;
  auto line_of = [&](int p, int u) { return (uint32_t)(p * 128) + wave * 32 + (uint32_t)u * 8 + grp; };
  // Tile t of block j: byte offset into a rank buffer, bytes and lines.
  auto tile_off = [&](int j) {
    uint64_t lo, hi;
    tile_range(g, block_len(g, (uint64_t)j), t, &lo, &hi);
    return (block_lo(g, (uint64_t)j) + lo) * es;
  };
  auto tile_bytes = [&](int j) {
    uint64_t lo, hi;
    tile_range(g, block_len(g, (uint64_t)j), t, &lo, &hi);
    return (uint32_t)((hi - lo) * es);
  };
  const uint64_t slot_stride = uniform64(g.slot_lines * g.line_bytes);
  const char* tile_lines = a.lines + uniform64(t * g.tile_lines * g.line_bytes);
  auto slot = [&](uint64_t sidx, uint32_t nb) {
    return make_rsrc(tile_lines + sidx * slot_stride, (uint32_t)cdiv(nb, LL128_DATA) * LL128_LINE);
  };
  const uint64_t nn = (uint64_t)n * n;

  // Step 0's first pass loads go out with the epoch.
  uint4 sp[MAX_RANKS][U_C128];
  auto load_send = [&](int p) {
#pragma unroll
    for (int j = 0; j < MAX_RANKS; ++j) {
      if (j >= n) break;
      if (j == r) continue;
      const Rsrc src = make_rsrc(a.in[r] + tile_off(j), tile_bytes(j));
#pragma unroll
      for (int u = 0; u < U_C128; ++u) sp[j][u] = load_piece_bounded<DT, WORDS>(src, line_of(p, u) * LL128_DATA + 16 * q, full);
    }
  };
  auto store_send = [&](int p) {
#pragma unroll
    for (int j = 0; j < MAX_RANKS; ++j) {
      if (j >= n) break;
      if (j == r) continue;
      const Rsrc dst = slot((uint64_t)r * n + j, tile_bytes(j));
#pragma unroll
      for (int u = 0; u < U_C128; ++u)
        cst16(dst, line_of(p, u) * LL128_LINE + 16 * q, full ? sp[j][u] : make_uint4(sp[j][u].x, sp[j][u].y, 0, 0));
    }
  };
  load_send(0);
  if (threadIdx.x == 0) {
    const uint64_t e = __hip_atomic_load(&a.ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ab = ld_u32(&a.ctl->abort);
    s_epoch = e;
    s_abort = ab;
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t epoch = uniform64(s_epoch);
  const bool aborted = uniform(s_abort) != 0;
  // The flag word: low half (calls mod (2^32 - 1)) + 1, never 0, so that a
  // line still holding its payload-first zero flag word never passes; high
  // half calls div (2^32 - 1).  One value per call; the receives compare the
  // low half (as LL's 4-byte flags, it repeats after 2^32 - 1 calls).
  const uint2 flag2 = make_uint2((uint32_t)(epoch % 0xffffffffull) + 1u, (uint32_t)(epoch / 0xffffffffull));
  uint32_t finished = 0, counted = 0;
  const int passes = (int)cdiv(g.tile * es, LL128_COLOCATED_PASS);  // at most PASSES (launch_collective)
  if (!aborted) {
    // step 0: send
    store_send(0);
#pragma unroll
    for (int p = 1; p < PASSES; ++p) {
      if (p >= passes) break;
      load_send(p);
      store_send(p);
    }
    wait_mem();
    if (!withheld(a, 0, r)) {
#pragma unroll
      for (int j = 0; j < MAX_RANKS; ++j) {
        if (j >= n) break;
        if (j == r) continue;
        const Rsrc dst = slot((uint64_t)r * n + j, tile_bytes(j));
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
          for (int u = 0; u < U_C128; ++u)  // lane 7 of each group: its line's flag word
            cst8(dst, q == 7 ? line_of(p, u) * LL128_LINE + LL128_DATA : 0x7ffffff0u, flag2);
      }
    }
    wait_mem();
    if (blockIdx.x == 0) counted = ld_u32(&a.ctl->done);
    // A wait over the flag words of `slots` (slot index per peer, lines of
    // the tile of that peer's block) of pass p, every peer and line at once.
    // Only the low half of each flag word is read (flag2.x, never 0).
    // Waiting on every pass's flags at once saved a round trip per step but
    // re-read the flags of the later pass at every failed poll (t=512: 3 %
    // faster, 1.4 times the bytes).
    uint32_t fl[MAX_RANKS][U_C128];
    auto wait_flags = [&](int p, auto slot_of, auto nb_of, int step) -> bool {
      auto load = [&]() {
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          if (i == r) continue;
          const Rsrc src = slot(slot_of(i), nb_of(i));
#pragma unroll
          for (int u = 0; u < U_C128; ++u)
            fl[i][u] = __builtin_amdgcn_raw_buffer_load_b32(src, line_of(p, u) * LL128_LINE + LL128_DATA, 0, CPOL_SC1);
        }
      };
      auto seen = [&]() {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          if (i == r) continue;
          const uint32_t nl = (uint32_t)cdiv(nb_of(i), LL128_DATA);
#pragma unroll
          for (int u = 0; u < U_C128; ++u) ok = ok && (line_of(p, u) >= nl || fl[i][u] == flag2.x);
        }
        return ok;
      };
      load();
      if (seen()) return true;
      PollClock clock;
      uint32_t level = 0;
      while (true) {
        poll_sleep(level);
        load();
        if (seen()) return true;
        const int st = clock.tick(a);
        if (st == POLL_ABORTED) { note_blocked(a.ctl, step, r); return false; }
        if (st == POLL_TIMED_OUT) { raise_timeout(a.ctl, step, r); return false; }
      }
    };
    // step 1: gather, sum, keep and publish block r's tile
    bool ok = true;
    const uint32_t nb_r = tile_bytes(r);
    const Rsrc own_in = make_rsrc(a.in[r] + tile_off(r), nb_r);
    const Rsrc own_out = make_rsrc(a.out[r] + tile_off(r), nb_r);
    const Rsrc pub = slot(nn + r, nb_r);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      if (p >= passes || !ok) break;
      uint4 mine[U_C128];
#pragma unroll
      for (int u = 0; u < U_C128; ++u) mine[u] = load_piece_bounded<DT, WORDS>(own_in, line_of(p, u) * LL128_DATA + 16 * q, full);
      ok = wait_flags(p, [&](int i) { return (uint64_t)i * n + r; }, [&](int) { return nb_r; }, 1);
      if (!ok) break;
      uint4 pv[MAX_RANKS][U_C128];
#pragma unroll
      for (int i = 0; i < MAX_RANKS; ++i) {
        if (i >= n) break;
        if (i == r) continue;
        const Rsrc src = slot((uint64_t)i * n + r, nb_r);
#pragma unroll
        for (int u = 0; u < U_C128; ++u) pv[i][u] = cld16(src, line_of(p, u) * LL128_LINE + 16 * q);
      }
#pragma unroll
      for (int u = 0; u < U_C128; ++u) {
        Vec<DT> acc;
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          const Vec<DT> x = Vec<DT>::widen(i == r ? mine[u] : pv[i][u]);
          if (i == 0) acc = x; else acc.add(x);
        }
        const uint4 res = acc.narrow();
        store_piece_bounded<DT, WORDS>(own_out, line_of(p, u) * LL128_DATA + 16 * q, full, res);
        cst16(pub, line_of(p, u) * LL128_LINE + 16 * q, full ? res : make_uint4(res.x, res.y, 0, 0));
      }
    }
    if (ok) {
      wait_mem();
      if (!withheld(a, 1, r)) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
          for (int u = 0; u < U_C128; ++u)
            cst8(pub, q == 7 ? line_of(p, u) * LL128_LINE + LL128_DATA : 0x7ffffff0u, flag2);
      }
      wait_mem();
    }
    // step 2: every other block's sum
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      if (p >= passes || !ok) break;
      ok = wait_flags(p, [&](int j) { return nn + j; }, [&](int j) { return tile_bytes(j); }, 2);
      if (!ok) break;
      uint4 pv[MAX_RANKS][U_C128];
#pragma unroll
      for (int j = 0; j < MAX_RANKS; ++j) {
        if (j >= n) break;
        if (j == r) continue;
        const Rsrc src = slot(nn + j, tile_bytes(j));
#pragma unroll
        for (int u = 0; u < U_C128; ++u) pv[j][u] = cld16(src, line_of(p, u) * LL128_LINE + 16 * q);
      }
#pragma unroll
      for (int j = 0; j < MAX_RANKS; ++j) {
        if (j >= n) break;
        if (j == r) continue;
        const Rsrc dst = make_rsrc(a.out[r] + tile_off(j), tile_bytes(j));
#pragma unroll
        for (int u = 0; u < U_C128; ++u) store_piece_bounded<DT, WORDS>(dst, line_of(p, u) * LL128_DATA + 16 * q, full, pv[j][u]);
      }
    }
    finished = 3;
  } else if (blockIdx.x == 0) {
    counted = ld_u32(&a.ctl->done);
  }
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&a.ctl->diag[5], (uint64_t)finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0) advance_epoch(a, epoch, counted);
  }
}

// Colocated LL two-shot (a.colocate, make_geometry's rule): workgroup b is
// rank r = b % N on tile t = b / N of every block, with the LL128 two-shot's
// steps and staging slots.  An LL line carries its flag in the same 8-byte
// store as its payload word, so a line is whole once its flag reads new:
// no step waits between payload and flag, and a receive is one round trip
// per round of W words a thread, each poll reloading every line of the round.
//   step 0: rank r's tile t of every other block j goes out as lines to
//           slot r*N + j (owner j);
//   step 1: owner r sums tile t of its block in rank order -- its own input
//           and the N-1 ranks' lines of slot i*N + r -- keeps the sum and
//           publishes it as lines to slot N*N + r;
//   step 2: rank r copies every other owner's published tile t into its
//           output.
// In place is safe: only this workgroup reads or writes tile t of rank r's
// buffer, and each of its writes follows the reads of the same bytes.
// WORDS: every tile holds whole words (an even bf16 count, 16-byte aligned
// buffers), so bf16 moves a word per access; otherwise two halves, so an odd
// count's last element is exact.
template <int DT, int W, bool WORDS>
__device__ __forceinline__ void colocated_twoshot_ll(const KArgs& a) {
  __shared__ uint64_t s_epoch;
  __shared__ uint32_t s_abort;
  const Geometry& g = a.g;
  const int n = g.nranks;
  const int r = (int)uniform(blockIdx.x % (uint32_t)n);
  const uint64_t t = uniform(blockIdx.x / (uint32_t)n);
  constexpr int es = Elem<DT>::size;
  constexpr bool HALVES = es == 2 && !WORDS;
  auto tile_off = [&](int j) {
    uint64_t lo, hi;
    tile_range(g, block_len(g, (uint64_t)j), t, &lo, &hi);
    return (block_lo(g, (uint64_t)j) + lo) * es;
  };
  auto tile_bytes = [&](int j) {
    uint64_t lo, hi;
    tile_range(g, block_len(g, (uint64_t)j), t, &lo, &hi);
    return (uint32_t)((hi - lo) * es);
  };
  const uint64_t slot_stride = uniform64(g.slot_lines * g.line_bytes);
  const char* tile_lines = a.lines + uniform64(t * g.tile_lines * g.line_bytes);
  auto slot = [&](uint64_t sidx, uint32_t nb) { return make_rsrc(tile_lines + sidx * slot_stride, cdiv(nb, 4) * 8); };
  const uint64_t nn = (uint64_t)n * n;
  // Word u of round `it` of this thread: byte offset in a tile.
  auto woff = [&](int it, int u) { return 4 * (threadIdx.x + (uint32_t)(it * W + u) * WG_THREADS); };
  // Bounded accesses: bytes past a tile read as 0 and are not written.
  auto ld_w = [&](Rsrc src, uint32_t off) -> uint32_t {
    if constexpr (HALVES)
      return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src, off, 0, 0) |
             ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src, off + 2, 0, 0) << 16);
    else
      return __builtin_amdgcn_raw_buffer_load_b32(src, off, 0, 0);
  };
  auto st_w = [&](Rsrc dst, uint32_t off, uint32_t v) {
    if constexpr (HALVES) {
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, dst, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v >> 16), dst, off + 2, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(v, dst, off, 0, 0);
    }
  };
  const int rounds = (int)cdiv(g.tile * es, (uint64_t)W * WG_THREADS * 4);

  // Step 0's first round of loads goes out with the epoch.
  uint32_t sp[MAX_RANKS][W];
  auto load_send = [&](int it) {
#pragma unroll
    for (int j = 0; j < MAX_RANKS; ++j) {
      if (j >= n) break;
      if (j == r) continue;
      const Rsrc src = make_rsrc(a.in[r] + tile_off(j), tile_bytes(j));
#pragma unroll
      for (int u = 0; u < W; ++u) sp[j][u] = ld_w(src, woff(it, u));
    }
  };
  load_send(0);
  if (threadIdx.x == 0) {
    const uint64_t e = __hip_atomic_load(&a.ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ab = ld_u32(&a.ctl->abort);
    s_epoch = e;
    s_abort = ab;
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t epoch = uniform64(s_epoch);
  const bool aborted = uniform(s_abort) != 0;
  const uint32_t flag = (uint32_t)(epoch % 0xffffffffull) + 1u;
  uint32_t finished = 0, counted = 0;
  if (!aborted) {
    // step 0: send
    const bool send = !withheld(a, 0, r);
    for (int it = 0; it < rounds; ++it) {
      if (it) load_send(it);
      if (!send) continue;
#pragma unroll
      for (int j = 0; j < MAX_RANKS; ++j) {
        if (j >= n) break;
        if (j == r) continue;
        const Rsrc dst = slot((uint64_t)r * n + j, tile_bytes(j));
#pragma unroll
        for (int u = 0; u < W; ++u) cst8(dst, 2 * woff(it, u), make_uint2(sp[j][u], flag));
      }
    }
    // The peers send at about the same time: polls issued before this
    // workgroup's own lines have landed mostly come back unwritten.
    wait_mem();
    if (blockIdx.x == 0) counted = ld_u32(&a.ctl->done);
    // Every line of round `it` of the N-1 peers' slots (slot_of(i), tile
    // bytes nb_of(i)), polled until all are written.
    uint2 got[MAX_RANKS][W];
    auto receive = [&](int it, auto slot_of, auto nb_of, int step) -> bool {
      auto load = [&]() {
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          if (i == r) continue;
          const Rsrc src = slot(slot_of(i), nb_of(i));
#pragma unroll
          for (int u = 0; u < W; ++u) got[i][u] = cld8(src, 2 * woff(it, u));
        }
      };
      auto seen = [&]() {  // lanes past a tile read zeros and count as written
        bool ok = true;
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          if (i == r) continue;
          const uint32_t nb = nb_of(i);
#pragma unroll
          for (int u = 0; u < W; ++u) ok = ok && (woff(it, u) >= nb || got[i][u].y == flag);
        }
        return ok;
      };
      load();
      if (seen()) return true;
      PollClock clock;
      uint32_t level = 0;
      while (true) {
        poll_sleep(level);
        load();
        if (seen()) return true;
        const int st = clock.tick(a);
        if (st == POLL_ABORTED) { note_blocked(a.ctl, step, r); return false; }
        if (st == POLL_TIMED_OUT) { raise_timeout(a.ctl, step, r); return false; }
      }
    };
    // step 1: gather, sum, keep and publish block r's tile
    bool ok = true;
    const uint32_t nb_r = tile_bytes(r);
    const Rsrc own_in = make_rsrc(a.in[r] + tile_off(r), nb_r);
    const Rsrc own_out = make_rsrc(a.out[r] + tile_off(r), nb_r);
    const Rsrc pub = slot(nn + r, nb_r);
    const bool publish = !withheld(a, 1, r);
    for (int it = 0; it < rounds && ok; ++it) {
      uint32_t mine[W];
#pragma unroll
      for (int u = 0; u < W; ++u) mine[u] = ld_w(own_in, woff(it, u));
      ok = receive(it, [&](int i) { return (uint64_t)i * n + r; }, [&](int) { return nb_r; }, 1);
      if (!ok) break;
#pragma unroll
      for (int u = 0; u < W; ++u) {
        Word<DT> acc;
#pragma unroll
        for (int i = 0; i < MAX_RANKS; ++i) {
          if (i >= n) break;
          const Word<DT> x = Word<DT>::widen(i == r ? mine[u] : got[i][u].x);
          if (i == 0) acc = x; else acc.add(x);
        }
        const uint32_t res = n > 1 ? acc.narrow() : mine[u];
        st_w(own_out, woff(it, u), res);
        if (publish) cst8(pub, 2 * woff(it, u), make_uint2(res, flag));
      }
    }
    if (ok) wait_mem();
    // step 2: every other block's sum
    for (int it = 0; it < rounds && ok; ++it) {
      ok = receive(it, [&](int j) { return nn + j; }, [&](int j) { return tile_bytes(j); }, 2);
      if (!ok) break;
#pragma unroll
      for (int j = 0; j < MAX_RANKS; ++j) {
        if (j >= n) break;
        if (j == r) continue;
        const Rsrc dst = make_rsrc(a.out[r] + tile_off(j), tile_bytes(j));
#pragma unroll
        for (int u = 0; u < W; ++u) st_w(dst, woff(it, u), got[j][u].x);
      }
    }
    finished = 3;
  } else if (blockIdx.x == 0) {
    counted = ld_u32(&a.ctl->done);
  }
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&a.ctl->diag[5], (uint64_t)finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0) advance_epoch(a, epoch, counted);
  }
}

template <int DT, int W, bool WORDS>
__global__ __launch_bounds__(WG_THREADS) void colocated_twoshot_ll_kernel(KArgs a) {
  warm_kernel_args();
  colocated_twoshot_ll<DT, W, WORDS>(a);
}

template <int DT, int PASSES, bool WORDS>
__global__ __launch_bounds__(WG_THREADS) void colocated_twoshot_kernel(KArgs a) {
  warm_kernel_args();
  colocated_twoshot_ll128<DT, PASSES, WORDS>(a);
}

// Small LL / LL128 one-shots (a.colocate) run in a kernel of their own: the
// LL send holds a whole tile in registers, which in the ticketed kernel
// would have cut the workgroups per CU of every LL one-shot call.
template <int DT, int PROTO, int PASSES>
__global__ __launch_bounds__(WG_THREADS) void colocated_kernel(KArgs a) {
  warm_kernel_args();
  colocated_oneshot<DT, PROTO, PASSES>(a);
}

template <int DT, int PROTO, int KIND>
__global__ __launch_bounds__(WG_THREADS) void collective_kernel(KArgs a) {
  warm_kernel_args();
  if constexpr (never_waits<PROTO, KIND>()) {
    // When the grid covers every ticket at once, tasks that never wait need
    // neither the counter nor its re-arming: workgroup b runs its own
    // tickets and the data loads go out at once.  Such a call neither reads
    // the abort word nor moves the epoch; it cannot block, and it writes no
    // flag that a later call could mistake for its own.
    if (a.fixed && !(KIND == K_ONESHOT && a.g.in_place)) {
      uint64_t first = (uint64_t)blockIdx.x * a.batch;
      if (a.by_die) first = die_ticket(blockIdx.x, a.by_die);  // the N programs of a tile on one die
      for (uint32_t i = 0; i < a.batch; ++i) {
        if (first + i >= a.g.ntasks) break;
        const Task k = decode(a.g, (uint32_t)(first + i));
        if (k.phase != PH_NONE) run_task<DT, PROTO, KIND>(a, k, 0);
      }
      return;
    }
  }
  __shared__ uint64_t s_epoch;
  __shared__ uint32_t s_ticket;
  // A call that starts with the abort word set (an earlier call's latched
  // error) runs nothing.  An abort raised during the call is seen by the
  // waits, so the fetches below need not read it: the first fetch then goes
  // out together with these two loads, one round trip for all three.  The
  // loaded values reach LDS only after the fetch is issued: a store of the
  // epoch to LDS right after its load made the compiler wait out each load
  // in turn (three round trips before the first task).
  uint32_t aborted = 0;
  uint64_t epoch0 = 0;
  if (threadIdx.x == 0) {
    epoch0 = __hip_atomic_load(&a.ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    aborted = ld_u32(&a.ctl->abort);
  }
  const uint32_t ntasks = (uint32_t)a.g.ntasks;
  const uint32_t batch = a.batch;
  // When the grid's first fetches cover every ticket, each workgroup
  // fetches once: a second fetch could only come back empty.
  const bool one_fetch = (uint64_t)gridDim.x * batch >= (uint64_t)ntasks;
  uint32_t finished = 0;  // tasks this workgroup ran (diagnostics)
  bool more = true;
  while (more) {
    // Every ticket, the first included, comes from the shared counter, so a
    // workgroup takes work only once it is running.  Handing out the first
    // batch by workgroup index instead deadlocks whenever fewer workgroups
    // fit on the GPU than the occupancy estimate says: the running ones then
    // take every later ticket and wait on tickets held by workgroups that
    // cannot be dispatched until one of them exits.
    // By die (tasks that never wait, a.by_die): each die draws from its own
    // counter the ticket indices of its share (die_ticket), so the N
    // programs sharing a tile run on one die.  Every die has workgroups
    // (the grid is a multiple of XCDS), so every share is drawn.
    if (threadIdx.x == 0) {
      uint32_t* counter = &a.ctl->ticket;
      if (never_waits<PROTO, KIND>() && a.by_die) counter = &a.ctl->die_next[blockIdx.x % (uint32_t)XCDS];
      const uint32_t t = __hip_atomic_fetch_add(counter, batch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_epoch = epoch0;
      s_ticket = aborted ? 0xffffffffu : t;
    }
    __syncthreads();
    // Broadcast through readfirstlane so every branch below is a scalar
    // (workgroup-uniform) branch: barriers inside tasks then always sit in
    // uniform control flow.
    const uint32_t first = uniform(s_ticket);
    const uint64_t epoch = uniform64(s_epoch);
    __syncthreads();
    // A batch of consecutive tickets, run in order: the smallest unfinished
    // ticket always belongs to a running workgroup that has finished its
    // earlier tickets, so batching keeps the schedule deadlock-free.
    if (never_waits<PROTO, KIND>() && a.by_die) {
      // A die's share in increasing ticket order: past the last ticket,
      // every later index of the share is past it too.
      for (uint32_t i = 0; i < batch; ++i) {
        const uint64_t tk = first == 0xffffffffu
                                ? ntasks
                                : die_ticket((uint32_t)((uint64_t)(first + i) * XCDS + blockIdx.x % (uint32_t)XCDS),
                                             a.by_die);
        if (tk >= ntasks) { more = false; break; }
        const Task k = decode(a.g, (uint32_t)tk);
        if (k.phase != PH_NONE) run_task<DT, PROTO, KIND>(a, k, epoch);
        ++finished;
        __syncthreads();
      }
      continue;
    }
    for (uint32_t i = 0; i < batch; ++i) {
      if (first >= ntasks || ntasks - first <= i) { more = false; break; }
      const Task k = decode(a.g, first + i);
      if (k.phase != PH_NONE) run_task<DT, PROTO, KIND>(a, k, epoch);
      ++finished;
      // Reconverge every lane before the next task or ticket fetch, so
      // thread 0's fetch never shares a divergent path with a task's tail.
      __syncthreads();
    }
    // Tickets are handed out in increasing order: once a batch reaches the
    // end, every later fetch would come back empty.
    if (one_fetch || first >= ntasks || ntasks - first <= batch) more = false;
  }
  if (threadIdx.x == 0) finish_workgroup(a, finished);
}

// Clears a latched error (one thread).
__global__ void reset_kernel(Ctl* c) {
  c->abort = 0;
  c->err_code = 0;
  c->err_key = 0xffffffffu;
  c->diag[0] = 0;
}

// ============================================================== launching
using KernelFn = void (*)(KArgs);

template <int DT, int PROTO>
static KernelFn pick_kind(int kind) {
  switch (kind) {
    case K_ONESHOT: return collective_kernel<DT, PROTO, K_ONESHOT>;
    case K_TWOSHOT: return collective_kernel<DT, PROTO, K_TWOSHOT>;
    case K_RS_DIRECT: return collective_kernel<DT, PROTO, K_RS_DIRECT>;
    case K_AG_DIRECT: return collective_kernel<DT, PROTO, K_AG_DIRECT>;
    case K_RING: return collective_kernel<DT, PROTO, K_RING>;
    case K_TREE:
      if constexpr (PROTO == PROTO_SIMPLE) return collective_kernel<DT, PROTO, K_TREE>;
      return nullptr;
    default: return nullptr;
  }
}

template <int DT>
static KernelFn pick_proto(int proto, int kind) {
  if (kind == K_COPY) return collective_kernel<DT, PROTO_SIMPLE, K_COPY>;
  switch (proto) {
    case PROTO_SIMPLE: return pick_kind<DT, PROTO_SIMPLE>(kind);
    case PROTO_LL: return pick_kind<DT, PROTO_LL>(kind);
    case PROTO_LL128: return pick_kind<DT, PROTO_LL128>(kind);
    default: return nullptr;
  }
}

// Tiles of one pass take the one-pass kernels, larger ones (up to
// LL_COLOCATED_PASSES / LL128_COLOCATED_PASSES passes) the many-pass ones.
static KernelFn pick_colocated(int dtype, int proto, uint64_t tile_bytes) {
  constexpr int MP = (int)LL_COLOCATED_PASSES, MP128 = (int)LL128_COLOCATED_PASSES;
  const bool one = tile_bytes <= (proto == PROTO_LL ? LL_COLOCATED_TILE : LL128_COLOCATED_PASS);
  switch (dtype * 3 + proto) {
    case DT_F32 * 3 + PROTO_LL: return one ? colocated_kernel<DT_F32, PROTO_LL, 1> : colocated_kernel<DT_F32, PROTO_LL, MP>;
    case DT_F32 * 3 + PROTO_LL128:
      return one ? colocated_kernel<DT_F32, PROTO_LL128, 1> : colocated_kernel<DT_F32, PROTO_LL128, MP128>;
    case DT_BF16 * 3 + PROTO_LL: return one ? colocated_kernel<DT_BF16, PROTO_LL, 1> : colocated_kernel<DT_BF16, PROTO_LL, MP>;
    case DT_BF16 * 3 + PROTO_LL128:
      return one ? colocated_kernel<DT_BF16, PROTO_LL128, 1> : colocated_kernel<DT_BF16, PROTO_LL128, MP128>;
    case DT_I32 * 3 + PROTO_LL: return one ? colocated_kernel<DT_I32, PROTO_LL, 1> : colocated_kernel<DT_I32, PROTO_LL, MP>;
    case DT_I32 * 3 + PROTO_LL128:
      return one ? colocated_kernel<DT_I32, PROTO_LL128, 1> : colocated_kernel<DT_I32, PROTO_LL128, MP128>;
    default: return nullptr;
  }
}

// Colocated two-shots.  LL: rounds of 4 words a thread for tiles of one
// 4 KiB pass, of 8 for larger ones.  LL128: one or two passes per tile.
// bf16 a word at a time when `words` (an even element count).
static KernelFn pick_colocated_twoshot(int dtype, int proto, uint64_t tile_bytes, bool words) {
  if (proto == PROTO_LL) {
    const bool one = tile_bytes <= LL_COLOCATED_TILE;
    switch (dtype) {
      case DT_F32:
        return one ? colocated_twoshot_ll_kernel<DT_F32, U_LL, true> : colocated_twoshot_ll_kernel<DT_F32, 2 * U_LL, true>;
      case DT_BF16:
        if (words)
          return one ? colocated_twoshot_ll_kernel<DT_BF16, U_LL, true> : colocated_twoshot_ll_kernel<DT_BF16, 2 * U_LL, true>;
        return one ? colocated_twoshot_ll_kernel<DT_BF16, U_LL, false> : colocated_twoshot_ll_kernel<DT_BF16, 2 * U_LL, false>;
      case DT_I32:
        return one ? colocated_twoshot_ll_kernel<DT_I32, U_LL, true> : colocated_twoshot_ll_kernel<DT_I32, 2 * U_LL, true>;
      default: return nullptr;
    }
  }
  if (proto != PROTO_LL128) return nullptr;
  constexpr int MP = (int)LL128_COLOCATED_PASSES;
  const bool one = tile_bytes <= LL128_COLOCATED_PASS;
  switch (dtype) {
    case DT_F32: return one ? colocated_twoshot_kernel<DT_F32, 1, true> : colocated_twoshot_kernel<DT_F32, MP, true>;
    case DT_BF16:
      // Element by element a tile of two passes needs one workgroup per CU,
      // and its grid (256 workgroups) more than half of that: ticketed.
      if (words) return one ? colocated_twoshot_kernel<DT_BF16, 1, true> : colocated_twoshot_kernel<DT_BF16, MP, true>;
      return one ? colocated_twoshot_kernel<DT_BF16, 1, false> : nullptr;
    case DT_I32: return one ? colocated_twoshot_kernel<DT_I32, 1, true> : colocated_twoshot_kernel<DT_I32, MP, true>;
    default: return nullptr;
  }
}

static KernelFn pick_colocated_twoshot_simple(int dtype) {
  switch (dtype) {
    case DT_F32: return colocated_twoshot_simple_kernel<DT_F32>;
    case DT_BF16: return colocated_twoshot_simple_kernel<DT_BF16>;
    case DT_I32: return colocated_twoshot_simple_kernel<DT_I32>;
    default: return nullptr;
  }
}

// Every block and tile a whole number of words (rank buffers are 16-byte
// aligned, blocks and tiles whole vectors, so only the buffer's end can
// fall mid-word).
static bool word_clean(const KArgs& a) { return (a.g.total * (uint64_t)a.g.esize) % 4 == 0; }

KernelFn pick_kernel(int dtype, int proto, int kind) {
  switch (dtype) {
    case DT_F32: return pick_proto<DT_F32>(proto, kind);
    case DT_BF16: return pick_proto<DT_BF16>(proto, kind);
    case DT_I32: return pick_proto<DT_I32>(proto, kind);
    default: return nullptr;
  }
}

// Workgroups per CU a call runs by default.  Measured at N=8 (fractions of
// HBM peak, grid = this x 256 CUs; "all" = every workgroup that fits, 6-7
// per CU for most kernels):
//   per CU          2      3      4    all
//   ring 256 MiB  0.845  0.887  0.893  0.870
//   ring 25 MiB   0.786  0.800  0.628  0.579
//   int32 64 MiB  0.834  0.866  0.856  0.811
//   two-shot 256  0.799  0.856  0.877  0.876
//   LL128 5 MiB   126us  114us  175us  175us
// More resident workgroups than this only add polling and contention.
constexpr int DEFAULT_WG_PER_CU = 3;

// Workgroups of kernel f a call may run at once on `device` (the current
// device): those that fit (occupancy x CUs), at most DEFAULT_WG_PER_CU per
// CU.  Cached per (kernel, device); safe to call from several host threads.
int resident_workgroups(KernelFn f, int device) {
  struct Entry {
    KernelFn f;
    int device, count;
  };
  static std::mutex mu;
  static Entry seen[256];
  static int used = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (seen[i].f == f && seen[i].device == device) return seen[i].count;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)f, WG_THREADS, 0) != hipSuccess)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) cus = 1;
  if (per_cu < 1) per_cu = 1;
  static const int wg_per_cu = [] {
    const char* e = getenv("AR_WG_PER_CU");
    const int v = e ? atoi(e) : DEFAULT_WG_PER_CU;
    return v < 1 ? 1 : (v > 16 ? 16 : v);
  }();
  if (per_cu > wg_per_cu) per_cu = wg_per_cu;
  const int total = per_cu * cus;
  std::lock_guard<std::mutex> lock(mu);
  if (used < 256) seen[used++] = {f, device, total};
  return total;
}

bool debug_enabled() {
  static const bool on = [] {
    const char* e = getenv("AR_DEBUG");
    return e && *e && strcmp(e, "0") != 0;
  }();
  return on;
}

hipError_t launch_collective(const KArgs& a, int device, hipStream_t stream, uint32_t max_workgroups,
                             LaunchInfo* info) {
  KernelFn f = pick_kernel(a.g.dtype, a.g.proto, a.g.kind);
  if (!f) return hipErrorInvalidValue;
  uint64_t cap = (uint64_t)resident_workgroups(f, device);
  // A workgroup budget (NCCL's channel count) leaves the other CUs to
  // concurrent kernels.  The one-shot in-place barrier needs the N rank
  // programs of a tile resident together, so it never gets fewer than N.
  if (max_workgroups) cap = umin(cap, umax((uint64_t)max_workgroups, (uint64_t)a.g.nranks));
  KArgs b = a;
  // Tickets per fetch (pick_batch).  The one-shot in-place barrier waits on
  // LATER tickets of its group, so it must take them one at a time.
  const bool barrier = a.g.kind == K_ONESHOT && a.g.proto == PROTO_SIMPLE && a.g.in_place;
  static const int max_batch = [] {
    const char* e = getenv("AR_BATCH");
    const int v = e ? atoi(e) : 4;
    return v < 1 ? 1 : (v > 16 ? 16 : v);
  }();
  static const bool forced = getenv("AR_BATCH") != nullptr;
  b.batch = barrier ? 1u : (forced ? (uint32_t)max_batch : pick_batch(a.g, cap, (uint32_t)max_batch));
  uint64_t grid = umin(cdiv(a.g.ntasks, b.batch), cap);
  if (grid < 1) grid = 1;
  // Tasks that never wait, all handed out in the grid's first batch: no
  // counter round trip before the first load, none after the last store.
  const bool waits_free = a.g.kind == K_COPY ||
                          (a.g.proto == PROTO_SIMPLE && !barrier &&
                           (a.g.kind == K_ONESHOT || a.g.kind == K_RS_DIRECT || a.g.kind == K_AG_DIRECT));
  b.fixed = (waits_free && grid * b.batch >= a.g.ntasks) ? 1u : 0u;
  // A one-shot whose inputs exceed one die's L2: the N rank programs of a
  // tile re-read the same N input tiles, so they run on one die and share
  // its L2 (N=8 bf16 640 KiB per rank: 10.8 -> 6.9 us in a graph; 1 MiB
  // 19.9 -> 8.2; at most a few percent either way when the inputs fit).
  // The N receivers of a direct all-gather's shard tile likewise.  Both
  // number their tickets so that the N sharing a tile are consecutive.
  b.by_die = 0;
  const uint64_t rank_bytes = a.g.total * (uint64_t)a.g.esize;
  const bool shared_tiles =
      a.g.proto == PROTO_SIMPLE &&
      ((a.g.kind == K_ONESHOT && !a.g.in_place && oneshot_by_die(a.g.nranks, rank_bytes)) ||
       (a.g.kind == K_AG_DIRECT && allgather_by_die(a.g.nranks, rank_bytes)));
  const uint64_t G = (uint64_t)a.g.nranks;
  const uint64_t die_grid = XCDS * G * cdiv(cdiv(a.g.ntasks, G), XCDS);
  if (b.fixed && b.batch == 1 && shared_tiles && die_grid <= cap) {  // within a workgroup budget too
    grid = die_grid;
    b.by_die = (uint32_t)G;
  } else if (!b.fixed && shared_tiles && a.g.kind == K_ONESHOT && grid >= XCDS) {
    // Ticketed one-shots: a counter per die (a grid of whole dies, so each
    // has workgroups to draw its share).  N=8 graph or eager time, one
    // counter -> one per die: bf16 16 MiB 94.3 -> 78.0 us, fp32 32 MiB
    // 173.9 -> 126.0, 256 MiB 1625 -> 1457; N=4 fp32 64 MiB 141 -> 98.  The
    // all-gather gained nothing this way (up to 5 % slower at N=2).
    grid = grid / XCDS * XCDS;
    b.by_die = (uint32_t)a.g.nranks;
  }
  // One workgroup per (tile, rank) of a small line-protocol one-shot, in a
  // kernel of its own, when the budget lets them all be resident; otherwise
  // the ticketed schedule.
  b.colocate = 0;
  if (a.g.colocated && !a.rearm_errors) {
    const uint64_t tile_bytes = a.g.tile * (uint64_t)a.g.esize;
    KernelFn fc = a.g.kind != K_TWOSHOT           ? pick_colocated(a.g.dtype, a.g.proto, tile_bytes)
                  : a.g.proto == PROTO_SIMPLE ? pick_colocated_twoshot_simple(a.g.dtype)
                                              : pick_colocated_twoshot(a.g.dtype, a.g.proto, tile_bytes, word_clean(a));
    // At most half of what is resident: the N workgroups of a tile wait on
    // each other, and another kernel may hold part of the GPU.
    uint64_t ccap = fc ? (uint64_t)resident_workgroups(fc, device) / 2 : 0;
    if (max_workgroups) ccap = umin(ccap, umax((uint64_t)max_workgroups, (uint64_t)a.g.nranks));
    if (fc && a.g.tiles * (uint64_t)a.g.nranks <= ccap) {
      f = fc;
      b.colocate = 1;
      b.batch = 1;
      grid = a.g.tiles * (uint64_t)a.g.nranks;
    }
  }
  // One-shot out of place folds every term of a pass at once while its N
  // inputs are small; beyond that the same fold ran slower than one term at
  // a time.  Measured at N=8 (us, one term at a time -> fold): bf16 4 MiB per
  // rank 43.7 -> 38.9, 16 MiB 112.8 -> 105.3, 32 MiB 187.5 -> 221.2; fp32
  // 4 MiB 39.4 -> 38.2, 8 MiB 59.2 -> 61.3, 32 MiB 169.5 -> 227.6.  bf16
  // gains further (twice the widen/add/round work per byte to hide).  So:
  // N inputs of at most 128 MiB (bf16) or 32 MiB (4-byte types) -- those
  // figures predate the placement by die.  Placed by die (the N programs of
  // a tile share one L2), the fold wins at every size: N=8 fp32 25 MiB
  // 123.9 -> 100.4 us, 256 MiB 1450 -> 1327; bf16 256 MiB 1646 -> 1353.
  static const uint64_t fold_env = [] {
    const char* e = getenv("AR_ONESHOT_FOLD_MIB");
    return e ? (strtoull(e, nullptr, 10) << 20) : ~0ull;
  }();
  const uint64_t fold_max = fold_env != ~0ull ? fold_env : (a.g.esize == 2 ? 128ull << 20 : 32ull << 20);
  const bool fold_by_die = fold_env == ~0ull && b.by_die != 0;
  b.fold = (a.g.kind == K_ONESHOT && !a.g.in_place &&
            (fold_by_die || (uint64_t)a.g.nranks * a.g.total * (uint64_t)a.g.esize <= fold_max)) ? 1u : 0u;
  hipLaunchKernelGGL(f, dim3((unsigned)grid), dim3(WG_THREADS), 0, stream, b);
  if (info) {
    info->grid = (uint32_t)grid;
    info->batch = b.batch;
    info->counter_free = b.fixed | b.colocate;
    info->by_die = b.by_die;
  }
  return hipGetLastError();
}

hipError_t launch_reset(Ctl* c, hipStream_t stream) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, stream, c);
  return hipGetLastError();
}

}  // namespace ar
