// schedule.hpp -- geometry and task decoding of every collective schedule.
//
// Used by both the host (planning, byte accounting) and the device kernels
// (task decoding), so every function is host+device and pure integer math.
//
// A call runs as ONE kernel whose workgroups take "tasks" from a ticket
// counter.  A task is one rank program's work on one tile (a contiguous
// element range) at one step of its schedule.  Tickets are ordered so that
// every task a task waits on has a smaller ticket; since a workgroup only
// takes a ticket while it is running, the smallest unfinished ticket can
// always make progress and the kernel cannot deadlock whatever the number of
// resident workgroups (the one exception, the one-shot in-place barrier,
// needs N resident workgroups, which every launch provides).
//
// Schedules ("Collective communication: NCCL's algorithms and protocols, and
// custom all-reduce", section "Algorithms"; "NCCL collectives, ring
// all-reduce & launching TP/PP", section "Direct answer"):
//
//   K_ONESHOT   every rank program r reads all N inputs and sums them.
//   K_TWOSHOT   rank j sums block j over all ranks, then every other rank
//               copies block j's sum.
//   K_RS_DIRECT rank r sums slice r of every rank (reduce-scatter).
//   K_AG_DIRECT rank r copies shard j of every rank (all-gather).
//   K_RING      chain per (block, chunk loop, tile): N-1 reduce steps and/or
//               N-1 copy steps, each run by the receiving rank; tickets go
//               window by window, step by step inside a window.
//   K_TREE      double binary tree (all-reduce, Simple): half h of the
//               buffer goes up tree h (heap layout; tree 0 holds rank p at
//               position p, tree 1 rank N-1-p), every node adding its own
//               input and its children's partials, then the root's sum goes
//               back down; each tile's up tasks run leaves first and its
//               down tasks root first, the levels `lag` ticket groups apart.
//   K_COPY      a single rank: output = input.
//
// With LL / LL128 a transfer is lines written by the sender into staging
// memory and polled by the receiver; the tasks are split accordingly
// (publish / send tasks, then receive tasks).  Ticket groups interleave the
// phases with a lag of a few tiles so receivers rarely wait.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define AR_HD __host__ __device__ __forceinline__
#else
#define AR_HD inline
#endif

namespace ar {

enum Op { OP_ALLREDUCE = 0, OP_REDUCE_SCATTER = 1, OP_ALLGATHER = 2 };
enum Algo { ALGO_ONESHOT = 0, ALGO_TWOSHOT = 1, ALGO_RING = 2, ALGO_TREE = 3 };
enum Proto { PROTO_SIMPLE = 0, PROTO_LL = 1, PROTO_LL128 = 2 };
enum DType { DT_F32 = 0, DT_BF16 = 1, DT_I32 = 2 };
enum Kind { K_COPY = 0, K_ONESHOT = 1, K_TWOSHOT = 2, K_RS_DIRECT = 3, K_AG_DIRECT = 4, K_RING = 5, K_TREE = 6 };

constexpr int MAX_RANKS = 8;
constexpr int WG_THREADS = 256;
constexpr int LL_LINE = 8, LL_DATA = 4;
constexpr int LL128_LINE = 128, LL128_DATA = 120;

// Phases of a decoded task (what the rank program does on its tile).
enum Phase {
  PH_NONE = 0,    // empty task (tile beyond the data): nothing to do
  PH_COPY,        // K_COPY
  PH_FOLD,        // sum N sources into the output (one-shot, RS, two-shot shot 1)
  PH_GATHER,      // copy a finished block into the rank's output
  PH_SEND,        // LL/LL128: encode the rank's own input slice as lines
  PH_RECV_FOLD,   // LL/LL128: own input + N-1 peers' lines -> output (+ publish)
  PH_RECV_COPY,   // LL/LL128: lines -> output
  PH_RING,        // one step of a ring chain
  PH_TREE_UP,     // tree: own input + children's partials -> own output
  PH_TREE_DOWN    // tree: parent's sum -> own output
};

struct Geometry {
  int32_t op, algo, proto, dtype, kind;
  int32_t nranks, esize, in_place;
  int32_t steps;        // ring: steps per chain
  int32_t lag;          // phased kinds: tiles between phases
  uint64_t count;       // AR: elements per rank; RS: recvcount; AG: sendcount
  uint64_t total;       // elements of the block-partitioned buffer (AR: count; RS/AG: N*count)
  uint64_t block;       // elements per block
  uint64_t tile;        // elements per task tile
  uint64_t chunk;       // ring: elements per chunk loop
  uint64_t tiles;       // tiles per block (direct kinds, K_ONESHOT: per buffer) or per chunk (ring)
  uint64_t loops;       // ring: chunk loops per block
  uint64_t window;      // ring: chunk loops per ticket window (skew == 0)
  uint64_t skew;        // ring: 0 = windowed order; k >= 1 = order by loop + k*step
  uint64_t groups;      // phased kinds: ticket groups
  uint64_t per_group;   // phased kinds: tasks per group
  uint64_t ntasks;
  uint64_t line_bytes;  // 8 (LL), 128 (LL128), 0 (Simple)
  uint64_t tile_lines;  // lines reserved per tile in staging
  uint64_t slot_lines;  // lines reserved per staging slot
  uint64_t nslots;      // staging slots
  uint64_t nflags;      // Simple flags used
  int32_t colocated;    // the plan fits one workgroup per (tile, rank), no tickets (see make_geometry)
  int32_t pad;
};

struct Task {
  int32_t phase;
  int32_t rank;     // executing rank program
  int32_t peer;     // block owner / sender / source, by phase
  int32_t step;     // schedule step (ring) or phase step (0/1) for signals
  uint64_t block;   // block index
  uint64_t lo, hi;  // element range within the block (or buffer for K_ONESHOT/K_COPY)
  uint64_t tile;    // tile index within the block (or buffer)
  uint64_t chain;   // ring: chain index (flags, staging)
};

AR_HD uint64_t cdiv(uint64_t a, uint64_t b) { return b ? (a + b - 1) / b : 0; }
AR_HD uint64_t umin(uint64_t a, uint64_t b) { return a < b ? a : b; }
AR_HD uint64_t umax(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Block j of the partitioned buffer: [j*block, min((j+1)*block, total)).
AR_HD uint64_t block_lo(const Geometry& g, uint64_t j) { return umin(j * g.block, g.total); }
AR_HD uint64_t block_len(const Geometry& g, uint64_t j) {
  return umin((j + 1) * g.block, g.total) - block_lo(g, j);
}

// The GPU's dies (XCDs): workgroups are handed to them in turn, so
// workgroup b runs on die b % XCDS.
constexpr uint64_t XCDS = 8;

// Ticket of workgroup b in a grid that runs each group of G consecutive
// tickets on one die: group m goes to die m % XCDS, as workgroups
// XCDS (G (m / XCDS) + i) + m % XCDS, i < G.  Over a grid of
// XCDS G ceil(groups / XCDS) workgroups every ticket appears exactly once
// (the workgroups whose ticket lies past the last one run nothing).
AR_HD uint64_t die_ticket(uint32_t b, uint32_t G) {
  const uint32_t q = b / (uint32_t)XCDS;
  return ((uint64_t)(b % (uint32_t)XCDS) + XCDS * (uint64_t)(q / G)) * G + q % G;
}

// Tile k of an extent of `len` elements cut in tiles of g.tile: [lo, hi).
AR_HD void tile_range(const Geometry& g, uint64_t len, uint64_t k, uint64_t* lo, uint64_t* hi) {
  *lo = umin(k * g.tile, len);
  *hi = umin((k + 1) * g.tile, len);
}

// Ring: the p-th (loop, step) cell of a `loops` x `steps` grid, in one of
// two orders; both put a chain's step s-1 before its step s.
//
// skew == 0, windowed: loops are cut into windows of `window` loops; windows
//   are taken in order and, inside one, step by step (all loops of step 0,
//   then of step 1, ...).  Predecessors sit a whole window-step earlier.
// skew k >= 1, skewed diagonal: cells ordered by loop + k*step (then step).
//   Step s+1 of a loop follows step s after about k*steps cells, so data a
//   step writes is read again soon (while still in the device cache) and
//   chunks stream through the steps like a pipeline.
AR_HD uint64_t ring_cells_below(uint64_t key, uint64_t loops, uint64_t steps, uint64_t skew) {
  uint64_t n = 0;  // cells with loop + skew*step < key
  for (uint64_t s = 0; s < steps && skew * s < key; ++s) n += umin(key - skew * s, loops);
  return n;
}

AR_HD void ring_cell(uint64_t p, uint64_t loops, uint64_t steps, uint64_t window, uint64_t skew,
                     uint64_t* loop, uint64_t* step) {
  if (skew == 0) {
    const uint64_t per_window = steps * window;
    const uint64_t w = p / per_window, r = p % per_window;
    const uint64_t first = w * window;
    const uint64_t width = umin(window, loops - first);  // the last window may be narrower
    *step = r / width;
    *loop = first + r % width;
    return;
  }
  uint64_t lo = 0, hi = loops + skew * (steps - 1);  // largest key with cells_below(key) <= p
  while (hi - lo > 1) {
    const uint64_t mid = (lo + hi) / 2;
    if (ring_cells_below(mid, loops, steps, skew) <= p) lo = mid; else hi = mid;
  }
  const uint64_t key = lo;
  const uint64_t s_lo = key + 1 > loops ? (key + 1 - loops + skew - 1) / skew : 0;
  const uint64_t s = s_lo + (p - ring_cells_below(key, loops, steps, skew));
  *step = s;
  *loop = key - skew * s;
}

AR_HD int32_t rank_mod(int64_t x, int32_t n) { return (int32_t)(((x % n) + n) % n); }

// Rank r' in [0, n-1) mapped onto [0, n) skipping `skip`.
AR_HD int32_t skip_rank(int32_t rp, int32_t skip) { return rp + (rp >= skip ? 1 : 0); }

// Depth of heap position `pos` (the root is 0).
AR_HD uint64_t tree_depth(int32_t pos) {
  uint64_t d = 0;
  for (uint32_t x = (uint32_t)pos + 1; x > 1; x >>= 1) ++d;
  return d;
}

// Rank at heap position `pos` of tree 0 or tree 1.
AR_HD int32_t tree_rank(int32_t n, uint64_t tree, int32_t pos) { return tree == 0 ? pos : n - 1 - pos; }

// Decode ticket t of geometry g.
AR_HD Task decode(const Geometry& g, uint64_t t) {
  Task k;
  k.phase = PH_NONE;
  k.rank = 0; k.peer = 0; k.step = 0;
  k.block = 0; k.lo = 0; k.hi = 0; k.tile = 0; k.chain = 0;
  const int32_t n = g.nranks;
  const bool lines = g.proto != PROTO_SIMPLE;

  if (g.kind == K_COPY) {
    k.phase = PH_COPY;
    k.tile = t;
    tile_range(g, g.total, t, &k.lo, &k.hi);
    return k;
  }

  if (g.kind == K_TREE) {
    // A group holds one of each of the 4N-2 tasks of a tile: up on tree 0
    // (positions N-1..0), up on tree 1, down on tree 0 (positions 1..N-1),
    // down on tree 1.  With lag 0 group g is tile g.  Otherwise each task
    // belongs to a stage (up: D - depth, leaves first; down: D + depth) and
    // group g holds, for every stage st, the tasks of tile g - st*lag: a
    // task's inputs then come from about `lag` groups earlier.
    const uint64_t per_group = 4ull * n - 2;
    const uint64_t group = t / per_group, r = t % per_group;
    uint64_t tree;
    int32_t pos;
    bool up;
    if (r < 2ull * n) {
      tree = r / n;
      pos = n - 1 - (int32_t)(r % n);
      up = true;
    } else {
      const uint64_t d = r - 2ull * n;
      tree = d / (n - 1);
      pos = 1 + (int32_t)(d % (n - 1));
      up = false;
    }
    const uint64_t depth = tree_depth(pos), deepest = tree_depth(n - 1);
    const uint64_t stage = up ? deepest - depth : deepest + depth;
    const uint64_t shift = stage * (uint64_t)g.lag;
    if (group < shift || group - shift >= g.tiles) return k;  // no tile in this slot
    k.phase = up ? PH_TREE_UP : PH_TREE_DOWN;
    k.block = tree;
    k.peer = pos;
    k.rank = tree_rank(n, tree, pos);
    k.tile = group - shift;
    tile_range(g, block_len(g, tree), k.tile, &k.lo, &k.hi);
    if (k.hi <= k.lo) k.phase = PH_NONE;
    return k;
  }

  if (g.kind == K_RING) {
    const uint64_t per_cell = (uint64_t)n * g.tiles;
    const uint64_t p = t / per_cell, rem = t % per_cell;
    uint64_t loop, step;
    ring_cell(p, g.loops, (uint64_t)g.steps, g.window, g.skew, &loop, &step);
    const uint64_t j = rem / g.tiles, kk = rem % g.tiles;
    k.block = j;
    k.step = (int32_t)step;
    k.chain = (j * g.loops + loop) * g.tiles + kk;
    k.tile = loop * g.tiles + kk;
    const uint64_t blen = block_len(g, j);
    const uint64_t c_lo = umin(loop * g.chunk, blen), c_hi = umin((loop + 1) * g.chunk, blen);
    k.lo = umin(c_lo + kk * g.tile, c_hi);
    k.hi = umin(c_lo + (kk + 1) * g.tile, c_hi);
    if (k.hi > k.lo) k.phase = PH_RING;
    // executing rank of step s of block j (see the K_RING kernel for meaning)
    const int red = (g.op == OP_ALLGATHER) ? 0 : n - 1;
    const int first = lines ? 1 : 0;  // LL/LL128: step 0 puts the first block on the wire
    const int32_t s = (int32_t)step;
    if (g.op == OP_ALLGATHER) {
      k.rank = rank_mod((int64_t)j + s, n);                  // step 0: owner; s: receiver j+s
    } else if (s < first) {
      k.rank = rank_mod((int64_t)j + 1, n);                  // first sender of block j
    } else if (s - first < red) {
      k.rank = rank_mod((int64_t)j + 2 + (s - first), n);    // reduce receiver
    } else {
      k.rank = rank_mod((int64_t)j + 1 + (s - first - red), n);  // copy receiver
    }
    return k;
  }

  const uint64_t grp = (g.kind == K_ONESHOT && !lines) || (g.kind == K_RS_DIRECT && !lines) ||
                               (g.kind == K_AG_DIRECT && !lines)
                           ? 0 : t / g.per_group;
  if (g.kind == K_ONESHOT) {
    if (!lines) {  // tasks (tile, rank)
      k.tile = t / (uint64_t)n;
      k.rank = (int32_t)(t % (uint64_t)n);
      k.step = 0;
      tile_range(g, g.total, k.tile, &k.lo, &k.hi);
      if (k.hi > k.lo) k.phase = PH_FOLD;
      return k;
    }
    const uint64_t rem = t % g.per_group;  // [publish x N][receive x N]
    if (rem < (uint64_t)n) {
      k.rank = (int32_t)rem;
      k.tile = grp;
      if (grp < g.tiles) { tile_range(g, g.total, k.tile, &k.lo, &k.hi); if (k.hi > k.lo) k.phase = PH_SEND; }
    } else {
      k.rank = (int32_t)(rem - n);
      if (grp >= (uint64_t)g.lag && grp - g.lag < g.tiles) {
        k.tile = grp - g.lag;
        tile_range(g, g.total, k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_RECV_FOLD;
      }
    }
    return k;
  }

  if (g.kind == K_TWOSHOT) {
    const uint64_t rem = t % g.per_group;
    const uint64_t nn1 = (uint64_t)n * (n - 1);
    if (!lines) {  // [owner sums block j x N][rank r copies block j x N(N-1)]
      if (rem < (uint64_t)n) {
        k.block = rem; k.rank = (int32_t)rem; k.step = 0;
        if (grp < g.tiles) {
          k.tile = grp;
          tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
          if (k.hi > k.lo) k.phase = PH_FOLD;
        }
      } else {
        const uint64_t q = rem - n;
        k.block = q / (n - 1);
        k.rank = skip_rank((int32_t)(q % (n - 1)), (int32_t)k.block);
        k.peer = (int32_t)k.block; k.step = 1;
        if (grp >= (uint64_t)g.lag && grp - g.lag < g.tiles) {
          k.tile = grp - g.lag;
          tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
          if (k.hi > k.lo) k.phase = PH_GATHER;
        }
      }
      return k;
    }
    // lines: [send i->j x N(N-1)][owner j x N][rank r receives block j x N(N-1)]
    if (rem < nn1) {
      k.rank = (int32_t)(rem / (n - 1));                       // sender
      k.block = (uint64_t)skip_rank((int32_t)(rem % (n - 1)), k.rank);  // owner
      k.peer = (int32_t)k.block;
      if (grp < g.tiles) {
        k.tile = grp;
        tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_SEND;
      }
    } else if (rem < nn1 + n) {
      k.block = rem - nn1; k.rank = (int32_t)k.block;
      if (grp >= (uint64_t)g.lag && grp - g.lag < g.tiles) {
        k.tile = grp - g.lag;
        tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_RECV_FOLD;
      }
    } else {
      const uint64_t q = rem - nn1 - n;
      k.block = q / (n - 1);
      k.rank = skip_rank((int32_t)(q % (n - 1)), (int32_t)k.block);
      k.peer = (int32_t)k.block;
      if (grp >= 2 * (uint64_t)g.lag && grp - 2 * g.lag < g.tiles) {
        k.tile = grp - 2 * g.lag;
        tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_RECV_COPY;
      }
    }
    return k;
  }

  if (g.kind == K_RS_DIRECT) {
    if (!lines) {  // tasks (tile, owner)
      k.tile = t / (uint64_t)n;
      k.block = t % (uint64_t)n; k.rank = (int32_t)k.block;
      tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
      if (k.hi > k.lo) k.phase = PH_FOLD;
      return k;
    }
    const uint64_t rem = t % g.per_group;  // [send i->j x N(N-1)][owner j x N]
    const uint64_t nn1 = (uint64_t)n * (n - 1);
    if (rem < nn1) {
      k.rank = (int32_t)(rem / (n - 1));
      k.block = (uint64_t)skip_rank((int32_t)(rem % (n - 1)), k.rank);
      k.peer = (int32_t)k.block;
      if (grp < g.tiles) {
        k.tile = grp;
        tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_SEND;
      }
    } else {
      k.block = rem - nn1; k.rank = (int32_t)k.block;
      if (grp >= (uint64_t)g.lag && grp - g.lag < g.tiles) {
        k.tile = grp - g.lag;
        tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_RECV_FOLD;
      }
    }
    return k;
  }

  if (g.kind == K_AG_DIRECT) {
    if (!lines) {  // tasks (tile, shard j, receiver r)
      const uint64_t nn = (uint64_t)n * n;
      k.tile = t / nn;
      const uint64_t rem = t % nn;
      k.block = rem / n; k.peer = (int32_t)k.block;
      k.rank = (int32_t)(rem % n);
      tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
      if (k.hi > k.lo) k.phase = PH_GATHER;
      return k;
    }
    const uint64_t rem = t % g.per_group;  // [publish j x N][receive x N(N-1)]
    if (rem < (uint64_t)n) {
      k.block = rem; k.rank = (int32_t)rem; k.peer = (int32_t)rem;
      if (grp < g.tiles) {
        k.tile = grp;
        tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_SEND;
      }
    } else {
      const uint64_t q = rem - n;
      k.block = q / (n - 1);
      k.rank = skip_rank((int32_t)(q % (n - 1)), (int32_t)k.block);
      k.peer = (int32_t)k.block;
      if (grp >= (uint64_t)g.lag && grp - g.lag < g.tiles) {
        k.tile = grp - g.lag;
        tile_range(g, block_len(g, k.block), k.tile, &k.lo, &k.hi);
        if (k.hi > k.lo) k.phase = PH_RECV_COPY;
      }
    }
    return k;
  }
  return k;
}

// Lines needed for a payload of `bytes` under the geometry's protocol.
AR_HD uint64_t lines_for(const Geometry& g, uint64_t bytes) {
  if (g.proto == PROTO_LL) return cdiv(bytes, LL_DATA);
  if (g.proto == PROTO_LL128) return cdiv(bytes, LL128_DATA);
  return 0;
}

}  // namespace ar
