// plan.hpp -- host-side planning of one call: schedule kind, block / chunk /
// tile geometry, ticket counts, staging and flag needs, and the byte
// accounting reported by ar_plan_bytes.  Pure C++ (no HIP calls).
#pragma once

#include <stdint.h>

#include "schedule.hpp"
#include "tuning_table.hpp"

namespace ar {

inline uint64_t floor_pow2(uint64_t x) {
  uint64_t p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

inline uint64_t clampu(uint64_t x, uint64_t lo, uint64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

constexpr uint64_t DEFAULT_CHUNK_BYTES = 512 * 1024;
// Workgroups an MI355X keeps resident for these kernels (256 CUs x up to 8):
// the tickets between a task and its predecessor should exceed it.
constexpr uint64_t RESIDENT_HINT = 2048;
// Tasks between the levels of one tree tile: about the default grid (3
// workgroups on each of 256 CUs) plus a third.
constexpr uint64_t TREE_RESIDENT_HINT = 1024;
// Tasks a call of a never-waiting schedule may have and still run in one
// grid (the default grid is 3 workgroups on each of 256 CUs, 768), so that
// it launches without the ticket counter.
constexpr uint64_t FIXED_GRID_TASKS = 512;
// The L2 of one die (XCD; the dies are XCDS in schedule.hpp).
constexpr uint64_t XCD_L2_BYTES = 4ull << 20;
// A one-shot whose N inputs together exceed one die's L2 runs the N rank
// programs of each tile on one die (launch_collective), so the tile's
// inputs come into that die's L2 once and the other N-1 programs hit them.
inline bool oneshot_by_die(uint64_t nranks, uint64_t rank_bytes) { return nranks * rank_bytes > XCD_L2_BYTES; }
// Likewise the N receivers of each shard tile of a direct all-gather, once
// the N x S bytes they write reach 32 MiB (S = the full per-rank buffer).
// N=8 bf16 graph time, 5 MiB per rank 14.2 -> 9.7 us, 8 MiB 21.4 -> 14.8;
// N=4 16 MiB 21.3 -> 14.8; N=2 32 MiB 21.6 -> 17.2.  Below that the
// placement cost up to 10 % (N=4 5 MiB 5.8 -> 6.4).
inline bool allgather_by_die(uint64_t nranks, uint64_t rank_bytes) { return nranks * rank_bytes >= (32ull << 20); }
// Bytes that one step of a ring window moves over all ranks: an eighth of
// the 256 MB last-level cache (MALL), so a step's partials are still there
// when the next step reads them.  Measured at N=8 with 512 KiB chunks (loops
// per window: fraction of HBM peak): 256 MiB fp32 4: 0.79, 6: 0.89,
// 8: 0.925, 10: 0.88, 16: 0.885, 32: 0.74; int32 64 MiB 8: 0.874, 16: 0.862;
// reduce-scatter 256 MiB 8: 0.882, 16: 0.874.
constexpr uint64_t RING_WINDOW_BYTES = 32ull << 20;
constexpr uint64_t LL128_TILE_UNIT = 3840;  // 32 lines of 120 payload bytes: one wave pass
// A one-shot call over LL or LL128 whose tiles fit this many workgroups (one
// per tile and rank) runs each rank's send and receive of a tile in one
// workgroup, with no ticket counter: the N workgroups of a tile wait on each
// other, so the grid is kept well below what is resident at once
// (launch_collective allows at most half).  Their own send and receive keep
// the latency from growing with the grid.
constexpr uint64_t COLOCATED_WORKGROUPS = 256;
// A colocated LL tile is whole passes of a workgroup (4 words per thread,
// 4 KiB), at most LL_COLOCATED_PASSES of them; its send loads the whole tile
// with the call's first round trip.
constexpr uint64_t LL_COLOCATED_TILE = 4096;
constexpr uint64_t LL_COLOCATED_PASSES = 8;
// A colocated LL128 tile is whole workgroup passes of 128 lines (4 waves x
// 32 lines: 15 KiB of payload), at most LL128_COLOCATED_PASSES of them.
constexpr uint64_t LL128_COLOCATED_PASS = 4 * 3840;
constexpr uint64_t LL128_COLOCATED_PASSES = 2;
// Simple two-shots run one workgroup per (tile, rank) -- fold tile t of the
// rank's own block, signal, wait for the other blocks' tile t, copy them --
// when a block (S / N) is at least SIMPLE_COLOCATED_MIN_BLOCK and its tiles,
// spread over COLOCATED_WORKGROUPS / N, at most SIMPLE_COLOCATED_MAX_TILE.
// Measured at N = 2, 4, 8 (us per call, ticketed -> colocated): N=8 bf16
// 2 MiB 30.3 -> 16.6, 5 MiB 46.4 -> 26.9, 25 MiB 125.8 -> 98.5, 64 MiB
// 268 -> 249 (256 KiB tiles), 128 MiB 422 -> 495 (512 KiB: kept ticketed);
// blocks of 16 KiB 10.9 -> 14.1 (kept ticketed), 64 KiB 25.1 -> 14.3.
constexpr uint64_t SIMPLE_COLOCATED_MIN_BLOCK = 64ull << 10;
constexpr uint64_t SIMPLE_COLOCATED_MAX_TILE = 256ull << 10;
constexpr uint64_t LL128_ALIGN = 240;       // 2 lines: a multiple of 16 bytes and of 120 bytes

inline int esize_of(int dtype) { return dtype == DT_BF16 ? 2 : 4; }

// AR_ALGO_AUTO / AR_PROTO_AUTO in the C ABI.
constexpr int ALGO_AUTO = 4;
constexpr int PROTO_AUTO = 3;
constexpr uint64_t MALL_BYTES = 256ull << 20;

// Fitted time (us) of one call with S = `rank_bytes` per rank, from the
// measured cost table: t = alpha + S * gamma, alpha and gamma interpolated
// linearly in N between the rank counts measured (clamped outside them).
// The cache band is 0 when the call's inputs and outputs fit in the MALL
// (2 N S <= 256 MiB).  Reduce-scatter and all-gather use the all-reduce fits
// of the same algorithm and protocol when none of their own were measured.
// Negative when the table has nothing for this combination.
inline double predict_us(int op, int nranks, int esize, int algo, int proto, uint64_t rank_bytes) {
  const int band = 2ull * (uint64_t)nranks * rank_bytes <= MALL_BYTES ? 0 : 1;
  for (int pass = 0; pass < 2; ++pass) {
    const int o = pass == 0 ? op : OP_ALLREDUCE;
    int lo = -1, hi = -1;
    for (int i = 0; i < N_COST_FITS; ++i) {
      const CostFit& f = COST_FITS[i];
      if (f.op != o || f.esize != esize || f.algo != algo || f.proto != proto || f.band != band) continue;
      if (f.nranks <= nranks && (lo < 0 || f.nranks > COST_FITS[lo].nranks)) lo = i;
      if (f.nranks >= nranks && (hi < 0 || f.nranks < COST_FITS[hi].nranks)) hi = i;
    }
    if (lo < 0 && hi < 0) continue;
    if (lo < 0) lo = hi;
    if (hi < 0) hi = lo;
    const CostFit& a = COST_FITS[lo];
    const CostFit& b = COST_FITS[hi];
    const double w = b.nranks == a.nranks ? 0.0 : double(nranks - a.nranks) / double(b.nranks - a.nranks);
    const double alpha = a.alpha_us + w * (b.alpha_us - a.alpha_us);
    const double gamma = a.us_per_byte + w * (b.us_per_byte - a.us_per_byte);
    return alpha + gamma * (double)rank_bytes;
  }
  return -1.0;
}

// Resolve ALGO_AUTO / PROTO_AUTO to the candidate with the smallest fitted
// time (fixed choices are kept).  LL and LL128 are candidates only when
// `line_ok` (the message fits the communicator's line staging).  On ties, or
// with no fit at all, the earlier candidate wins: Simple before LL before
// LL128, one-shot before two-shot before ring before tree.  Returns false on
// a bad argument.
inline bool select_schedule(int op, int nranks, int dtype, uint64_t rank_bytes, int algo, int proto,
                            bool line_ok, int* out_algo, int* out_proto, double* out_us) {
  if (op < 0 || op > 2 || dtype < 0 || dtype > 2 || nranks < 1 || nranks > MAX_RANKS) return false;
  if (algo < 0 || algo > ALGO_AUTO || proto < 0 || proto > PROTO_AUTO) return false;
  int best_a = algo == ALGO_AUTO ? ALGO_ONESHOT : algo;
  int best_p = proto == PROTO_AUTO ? PROTO_SIMPLE : proto;
  double best_t = -1.0;
  for (int a = 0; a < 4; ++a) {
    if (algo != ALGO_AUTO && a != algo) continue;
    // reduce-scatter / all-gather: two-shot names the same direct schedule,
    // and the tree is an all-reduce schedule
    if (algo == ALGO_AUTO && op != OP_ALLREDUCE && (a == ALGO_TWOSHOT || a == ALGO_TREE)) continue;
    for (int p = 0; p < 3; ++p) {
      if (proto != PROTO_AUTO && p != proto) continue;
      if (proto == PROTO_AUTO && p != PROTO_SIMPLE && !line_ok) continue;
      if (a == ALGO_TREE && p != PROTO_SIMPLE) continue;  // the tree runs with Simple only
      const double t = predict_us(op, nranks, esize_of(dtype), a, p, rank_bytes);
      if (t < 0) continue;
      if (best_t < 0 || t < best_t) { best_t = t; best_a = a; best_p = p; }
    }
  }
  *out_algo = best_a;
  *out_proto = best_p;
  if (out_us) *out_us = best_t;
  return true;
}

// Tuning knobs (no effect on results): 0 keeps the built-in choice.
struct Tuning {
  uint64_t tile_bytes = 0;  // Simple tile size
  uint64_t line_tile_bytes = 0;  // LL / LL128 tile payload (LL128: rounded to whole wave passes)
  uint64_t ring_skew = 0;   // ring order: 0 windowed, k >= 1 skewed diagonal
  uint64_t ring_window = 0; // ring window (loops) for the windowed order
  bool ring_skew_set = false;
  uint64_t lag = 0;         // phased kinds: receiver groups behind their senders
  uint64_t coloc_tile_bytes = 0;  // Simple two-shot: largest colocated tile (0 with _set: never)
  bool coloc_tile_set = false;
};

// Tile size in bytes for a per-rank buffer of `rank_bytes`: aim for >= 128
// tiles per rank so a call spreads over the 256 CUs, within per-schedule
// bounds measured at N=8 fp32 (fractions of HBM peak, default grid):
//   ring, tree    32 KiB  (ring 256 MiB: 0.87 at 32 KiB, 0.79 at 64, 0.72 at 128)
//   two-shot      64 KiB from 64 MiB per rank (256 MiB: 0.91 against 0.86 at
//                 32 KiB), else 32 KiB (25 MiB: 0.59 against 0.56 at 64 KiB)
//   one-shot      128 KiB (each task reads N tiles; 256 MiB: 1.59 ms against
//                 1.63 at 64 KiB and 1.96 at 32 KiB); 16 KiB in place (the
//                 tile lives in registers)
//   RS direct     16 KiB (256 MiB: 0.72 against 0.62 at 128 KiB)
//   AG direct     16 KiB from 64 MiB per rank (256 MiB: 409 us against 467
//                 at 128 KiB), else 128 KiB: an all-gather has N^2 tasks per
//                 tile row, and with 16 KiB tiles at 8-32 MiB each fetch of
//                 the ticket counter covers one small tile (N=8 8 MiB: 65 us
//                 against 32 at 128 KiB; N=2 32 MiB: 65 against 29)
// LL up to 32 KiB; LL128 whole wave passes (3840 payload bytes each), up to
// 8 (30 KiB), one-shot 16, direct reduce-scatter 4.  Measured at N=8, 256 MiB
// fp32 (us, the earlier caps of 16 KiB and 4 passes -> these): LL128 two-shot
// 2737 -> 2356, ring 2362 -> 2311, all-gather 1042 -> 913, one-shot 4628 ->
// 4164 (4421 at 8 passes); LL two-shot 2767 -> 2569, ring 2995 -> 2883,
// all-gather 1113 -> 1066, one-shot 5542 -> 5378.  The reduce-scatter ran
// slower with larger tiles (LL128 1447 at 4 passes, 1549 at 8).  5 MiB bf16
// (tokens 512): two-shot LL128 89 -> 88, one-shot LL128 108 -> 96.  At
// N <= 4 the message-size sweep measured one-shot LL128 5-13 % and two-shot
// LL 1-11 % slower from 128 MiB with the larger tiles: there they keep 4
// passes and 16 KiB.
inline uint64_t simple_tile_cap(uint64_t rank_bytes, int kind, bool in_place) {
  uint64_t hi = 131072;
  if (kind == K_RING || kind == K_TREE) hi = 32768;
  if (kind == K_TWOSHOT) hi = rank_bytes >= (64ull << 20) ? 65536 : 32768;
  if (kind == K_RS_DIRECT) hi = 16384;
  if (kind == K_AG_DIRECT) hi = rank_bytes >= (64ull << 20) ? 16384 : 131072;
  if (kind == K_ONESHOT && in_place) hi = 16384;
  return hi;
}

inline uint64_t pick_tile_bytes(int proto, uint64_t rank_bytes, int kind, bool in_place, int nranks = 8) {
  const uint64_t want = floor_pow2(rank_bytes / 128 + 1);
  if (proto == PROTO_SIMPLE) {
    uint64_t cap = simple_tile_cap(rank_bytes, kind, in_place);
    // A one-shot placed by die keeps about 12 tiles of N inputs in flight
    // on each die: 64 KiB tiles beat 128 KiB there (N=8 fp32 256 MiB 1327
    // -> 1257 us, 25 MiB 100.1 -> 96.5; 32 KiB: 1274, 116.2).
    if (kind == K_ONESHOT && !in_place && oneshot_by_die((uint64_t)nranks, rank_bytes)) cap = umin(cap, 65536);
    return clampu(want, 4096, cap);
  }
  if (proto == PROTO_LL) return clampu(want, 4096, kind == K_TWOSHOT && nranks <= 4 ? 16384 : 32768);
  const uint64_t passes =
      kind == K_ONESHOT ? (nranks <= 4 ? 4 : 16) : (kind == K_RS_DIRECT ? 4 : 8);
  return LL128_TILE_UNIT * clampu(floor_pow2(want / LL128_TILE_UNIT + 1), 1, passes);
}

// Tickets a workgroup takes per fetch.  Every fetch is an atomic on one
// counter, which serializes at about one per ~10 ns: a 256 MiB ring with
// 16 KiB tiles and one ticket per fetch spends more time in the counter than
// in HBM (0.43 of peak).  A fetch should cover about 64 KiB of tiles, and a
// workgroup should still see >= 4 fetches, so work stays balanced.
constexpr uint64_t BYTES_PER_FETCH = 65536;
inline uint32_t pick_batch(const Geometry& g, uint64_t resident, uint32_t max_batch) {
  const uint64_t tile_b = g.proto == PROTO_SIMPLE ? g.tile * (uint64_t)g.esize
                                                  : g.tile_lines * (uint64_t)g.line_bytes;
  uint64_t b = tile_b ? BYTES_PER_FETCH / tile_b : 1;
  b = clampu(b, 1, max_batch);
  const uint64_t spread = resident ? g.ntasks / (4 * resident) : 1;
  return (uint32_t)clampu(b, 1, spread > 0 ? spread : 1);
}

// Fill g for one call.  Returns false on an invalid combination.
inline bool make_geometry(int op, int algo, int proto, int dtype, int nranks, uint64_t count,
                          uint64_t chunk_bytes, int in_place, Geometry* out, const Tuning& tune = Tuning()) {
  if (nranks < 1 || nranks > MAX_RANKS) return false;
  if (op < 0 || op > 2 || algo < 0 || algo > 3 || proto < 0 || proto > 2 || dtype < 0 || dtype > 2)
    return false;
  Geometry g = {};
  g.op = op; g.algo = algo; g.proto = proto; g.dtype = dtype;
  g.nranks = nranks;
  g.esize = esize_of(dtype);
  g.in_place = in_place ? 1 : 0;
  g.count = count;
  g.lag = 2;
  const uint64_t n = (uint64_t)nranks, es = (uint64_t)g.esize, vec = 16 / es;
  g.line_bytes = proto == PROTO_LL ? LL_LINE : (proto == PROTO_LL128 ? LL128_LINE : 0);

  if (op == OP_ALLREDUCE) {
    g.total = count;
    g.block = cdiv(cdiv(count, n), vec) * vec;
  } else {
    g.total = n * count;
    g.block = count;
  }

  if (nranks == 1) {  // a single rank: its result is its own input
    g.kind = K_COPY;
    g.proto = PROTO_SIMPLE;
    g.line_bytes = 0;
    g.total = count;
    g.block = count;
    g.tile = pick_tile_bytes(PROTO_SIMPLE, count * es, K_COPY, false) / es;
    g.tiles = cdiv(count, g.tile);
    g.ntasks = (op == OP_ALLREDUCE && in_place) ? 0 : g.tiles;
    *out = g;
    return true;
  }

  if (algo == ALGO_TREE && (op != OP_ALLREDUCE || proto != PROTO_SIMPLE)) return false;  // all-reduce, Simple
  if (op == OP_ALLREDUCE)
    g.kind = algo == ALGO_ONESHOT ? K_ONESHOT
             : algo == ALGO_TWOSHOT ? K_TWOSHOT
             : algo == ALGO_TREE ? K_TREE : K_RING;
  else if (op == OP_REDUCE_SCATTER) g.kind = algo == ALGO_RING ? K_RING : K_RS_DIRECT;
  else g.kind = algo == ALGO_RING ? K_RING : K_AG_DIRECT;

  const bool lines = proto != PROTO_SIMPLE;
  const uint64_t rank_bytes = g.total * es;
  uint64_t tile_b = pick_tile_bytes(proto, rank_bytes, g.kind, in_place != 0, nranks);
  if (tune.tile_bytes && !lines && !(g.kind == K_ONESHOT && in_place))
    tile_b = clampu(tune.tile_bytes / 16 * 16, 4096, 512 * 1024);
  if (tune.line_tile_bytes && lines)
    tile_b = proto == PROTO_LL128 ? LL128_TILE_UNIT * clampu(tune.line_tile_bytes / LL128_TILE_UNIT, 1, 64)
                                  : clampu(tune.line_tile_bytes / 16 * 16, 1024, 256 * 1024);
  // Small one-shot calls over the line protocols run one workgroup per
  // (tile, rank) when they fit COLOCATED_WORKGROUPS workgroups.  Tiles are
  // whole workgroup passes (LL: 4 KiB, up to 8; LL128: 128 lines, up to 2):
  // the send loads the whole tile at once, the receive walks the passes in
  // turn.  Graph time at N=8, ticketed -> colocated: LL bf16 10 KiB 9.8 ->
  // 6.0 us, 640 KiB 50.7 -> 31.9; LL128 bf16 640 KiB 35.6 -> 24.0, fp32
  // 128 KiB 15.8 -> 8.8.
  // Line two-shots whose blocks exceed one pass likewise run one workgroup
  // per (tile, rank), a tile being tile t of every block.  LL, N=8 bf16,
  // graph time ticketed -> colocated: 80 KiB 20.7 -> 17.9 us, 640 KiB
  // 57.5 -> 23.2, 5 MiB 90.8 -> 66.2; N=2 640 KiB 19.0 -> 10.3.
  bool colocated = false;
  const bool coloc_kind = g.kind == K_ONESHOT || g.kind == K_TWOSHOT;
  if (lines && coloc_kind && !tune.line_tile_bytes && rank_bytes) {
    // Tiles are whole passes.  Rounding LL128 tiles to 32-line units
    // instead (more, partly filled workgroups) ran no faster: t=512 two-shot
    // 62.7 -> 63.4 us, t=8 one-shot 10.5 -> 12.0.  A two-shot whose blocks
    // fit one pass stays ticketed: each workgroup would then run the three
    // steps of its one tile in turn, where the ticketed schedule overlaps
    // them (LL128 t=1 15.9 -> 23.6 us, t=8 22.4 -> 25.2 when colocated; LL
    // t=1 13.7 -> 16.5).
    const uint64_t max_tiles = COLOCATED_WORKGROUPS / n;
    const uint64_t pass = proto == PROTO_LL ? LL_COLOCATED_TILE : LL128_COLOCATED_PASS;
    const uint64_t passes = proto == PROTO_LL ? LL_COLOCATED_PASSES : LL128_COLOCATED_PASSES;
    const uint64_t extent = g.kind == K_ONESHOT ? rank_bytes : g.block * es;
    const uint64_t need = cdiv(cdiv(extent, max_tiles), pass) * pass;
    if (need <= passes * pass && (g.kind == K_ONESHOT || extent > pass)) {
      tile_b = umax(need, pass);
      colocated = true;
    }
  }
  if (!lines && g.kind == K_TWOSHOT && !tune.tile_bytes && g.block) {
    const uint64_t max_tile = tune.coloc_tile_set ? tune.coloc_tile_bytes : SIMPLE_COLOCATED_MAX_TILE;
    const uint64_t block_b = g.block * es;
    const uint64_t need = cdiv(cdiv(block_b, COLOCATED_WORKGROUPS / n), 16) * 16;
    if (block_b >= SIMPLE_COLOCATED_MIN_BLOCK && need <= max_tile) {
      tile_b = need;
      colocated = true;
    }
  }
  // Tasks that never wait (Simple one-shot out of place, direct RS and AG)
  // skip the ticket counter when one grid covers them all.  A call that
  // would just miss that grid takes tiles large enough to fit in it: above
  // one grid every task costs a fetch of the shared counter, and the
  // serialized fetches set the time.  Measured at N=8 (us, before -> after):
  // all-gather 512 KiB per rank 27.9 -> 3.4, 2 MiB 30.1 -> 15.2, 8 MiB
  // 31.7 -> 24.2 (tiles up to the schedule's bound); reduce-scatter 32 MiB
  // N=2 44 -> 21, N=4 49 -> 33, N=8 68 -> 56 (64 KiB tiles); one-shot
  // 512 KiB 26.5 -> 6.1.  A one-shot task reads N tiles, and past 16 KiB
  // tiles the longer tasks cost more than the fetches save (8 MiB: 58 -> 92
  // with 128 KiB tiles), so one-shot tiles grow to 16 KiB at most and
  // reduce-scatter tiles to 64 KiB.  A one-shot placed by die (each tile's N
  // programs on one die, oneshot_by_die) takes tiles up to 128 KiB instead:
  // N=8 bf16 graph time, ticketed -> one grid by die: 2 MiB 28.5 -> 11.9 us,
  // 5 MiB 44.0 -> 23.9, 8 MiB 53.8 -> 35.3.
  if (!lines && !tune.tile_bytes &&
      ((g.kind == K_ONESHOT && !in_place) || g.kind == K_RS_DIRECT || g.kind == K_AG_DIRECT)) {
    const uint64_t per_row = g.kind == K_AG_DIRECT ? n * n : n;  // tasks per tile of every block
    const uint64_t extent_b = (g.kind == K_ONESHOT ? g.total : g.block) * es;
    const uint64_t rows = umax(1, FIXED_GRID_TASKS / per_row);
    const uint64_t need = cdiv(cdiv(extent_b, rows), 16) * 16;
    const uint64_t bound = g.kind == K_ONESHOT     ? (oneshot_by_die(n, rank_bytes) ? 131072 : 16384)
                           : g.kind == K_RS_DIRECT ? 65536
                                                   : simple_tile_cap(rank_bytes, g.kind, in_place != 0);
    if (need > tile_b && need <= bound) tile_b = need;
  }

  if (g.kind == K_RING) {
    uint64_t cb = chunk_bytes ? chunk_bytes : DEFAULT_CHUNK_BYTES;
    if (proto == PROTO_LL128) cb = (cb / LL128_ALIGN) * LL128_ALIGN;
    else cb = (cb / 16) * 16;
    if (cb == 0) cb = proto == PROTO_LL128 ? LL128_ALIGN : 16;
    // A chunk loop never reaches past a block: with blocks shorter than the
    // chunk, the tiles beyond the block would all be empty, yet each would
    // still cost a ticket at every step (an 8-byte call at N=8 took 14,336
    // tickets instead of 112).  Results do not depend on the chunk size.
    const uint64_t align = proto == PROTO_LL128 ? LL128_ALIGN : 16;
    const uint64_t block_b = cdiv(g.block * es, align) * align;
    if (block_b && cb > block_b) cb = block_b;
    tile_b = umin(tile_b, cb);
    g.chunk = cb / es;
    g.tile = tile_b / es;
    g.tiles = cdiv(g.chunk, g.tile);  // tiles per chunk loop
    g.loops = g.block ? cdiv(g.block, g.chunk) : 0;
    // window: the loops whose chunks one step of a window moves fit
    // RING_WINDOW_BYTES (for 512 KiB chunks at N=8: 8 loops)
    g.window = umax(1, umin(g.loops, RING_WINDOW_BYTES / (n * cb)));
    if (tune.ring_window) g.window = umax(1, umin(g.loops, tune.ring_window));
    g.skew = tune.ring_skew_set ? tune.ring_skew : 0;
    if (op == OP_ALLREDUCE) g.steps = lines ? 2 * nranks - 1 : 2 * (nranks - 1);
    else if (op == OP_REDUCE_SCATTER) g.steps = lines ? nranks : nranks - 1;
    else g.steps = nranks;
    g.ntasks = g.loops * (uint64_t)g.steps * n * g.tiles;
    g.nflags = lines ? 0 : n * g.loops * g.tiles;
    g.tile_lines = lines ? lines_for(g, tile_b) : 0;
    g.slot_lines = g.loops * g.tiles * g.tile_lines;
    g.nslots = lines ? n * (uint64_t)(g.steps - 1) : 0;
    *out = g;
    return true;
  }

  if (g.kind == K_TREE) {  // two halves: the N=2 block split
    g.block = cdiv(cdiv(count, 2), vec) * vec;
    g.tile = tile_b / es;
    g.tiles = cdiv(g.block, g.tile);
    g.per_group = 4ull * n - 2;
    // Levels of a tile `lag` groups apart, about one resident grid of tasks,
    // so a task's inputs are mostly ready when it starts.  When every task
    // fits in one grid there is no lag: the levels of a tile follow each
    // other directly (a lag would only stretch the chain of a small call).
    const uint64_t deepest = tree_depth(n - 1);
    g.lag = g.tiles * g.per_group <= TREE_RESIDENT_HINT
                ? 0
                : (int32_t)umax(1, umin(g.tiles, cdiv(TREE_RESIDENT_HINT, g.per_group)));
    g.groups = g.tiles + 2 * deepest * (uint64_t)g.lag;
    g.ntasks = g.groups * g.per_group;
    g.nflags = 2ull * g.tiles * n;
    *out = g;
    return true;
  }

  g.tile = tile_b / es;
  g.tile_lines = lines ? lines_for(g, tile_b) : 0;
  const uint64_t extent = (g.kind == K_ONESHOT) ? g.total : g.block;
  g.tiles = cdiv(extent, g.tile);
  // Receivers of tile g run `lag` groups after its senders: about one
  // resident grid of tasks in between, and at most a quarter of the tiles.
  // With the lag at the tile count, a small call's receivers all queued
  // behind its last sender: measured at N=8 bf16 (us, that lag -> a quarter
  // of the tiles or near it), two-shot Simple 5 MiB 56 -> 50, LL 512 KiB
  // 85 -> 63, LL128 5 MiB 104 -> 82-86; large calls keep the grid-sized lag
  // (two-shot LL128 32 MiB: 392 at 32 groups, 428-464 at 8-16).  One-shot
  // LL takes the same grid-sized lag (32 groups at N=8) although its groups
  // hold 2N tasks, not N^2: 5 MiB 122 us at 128 groups, 107 at 32; 32 MiB
  // 623 and 619.  One-shot LL128 keeps the 2N-task count (128 groups): at
  // 32 groups its 8 MiB call took 380 us against 184-190 at 64-128.
  const uint64_t per_group_hint = (g.kind == K_ONESHOT && proto == PROTO_LL128) ? 2 * n : n * n;
  g.lag = (int32_t)umax(1, umin(g.tiles / 4, cdiv(RESIDENT_HINT, per_group_hint)));
  if (tune.lag) g.lag = (int32_t)umax(1, umin(g.tiles, tune.lag));
  const uint64_t lag = (uint64_t)g.lag;
  switch (g.kind) {
    case K_ONESHOT:
      if (!lines) {
        g.ntasks = g.tiles * n;
        g.nflags = in_place ? g.tiles * n : 0;
      } else {
        g.per_group = 2 * n;
        g.groups = g.tiles ? g.tiles + lag : 0;
        g.nslots = n;
        g.colocated = colocated && g.tiles * n <= COLOCATED_WORKGROUPS ? 1 : 0;
      }
      break;
    case K_TWOSHOT:
      if (!lines) {
        g.per_group = n * n;
        g.groups = g.tiles ? g.tiles + lag : 0;
        g.nflags = n * g.tiles;
        g.colocated = colocated && g.tiles * n <= COLOCATED_WORKGROUPS ? 1 : 0;
      } else {
        g.per_group = n * (2 * n - 1);
        g.groups = g.tiles ? g.tiles + 2 * lag : 0;
        g.nslots = n * n + n;
        g.colocated = colocated && g.tiles * n <= COLOCATED_WORKGROUPS ? 1 : 0;
      }
      break;
    case K_RS_DIRECT:
      if (!lines) {
        g.ntasks = g.tiles * n;
      } else {
        g.per_group = n * n;
        g.groups = g.tiles ? g.tiles + lag : 0;
        g.nslots = n * n;
      }
      break;
    case K_AG_DIRECT:
      if (!lines) {
        g.ntasks = g.tiles * n * n;
      } else {
        g.per_group = n * n;
        g.groups = g.tiles ? g.tiles + lag : 0;
        g.nslots = n;
      }
      break;
    default:
      return false;
  }
  if (g.per_group) g.ntasks = g.groups * g.per_group;
  g.slot_lines = g.tiles * g.tile_lines;
  *out = g;
  return true;
}

inline uint64_t staging_bytes(const Geometry& g) { return g.nslots * g.slot_lines * g.line_bytes; }

// Byte accounting of one call: walk every task.  `link` has nranks entries.
struct Bytes {
  uint64_t rd = 0, wr = 0;
  uint64_t link[MAX_RANKS] = {};
};

inline Bytes account(const Geometry& g) {
  Bytes b;
  const int n = g.nranks;
  const uint64_t es = (uint64_t)g.esize;
  const bool lines = g.proto != PROTO_SIMPLE;
  for (uint64_t t = 0; t < g.ntasks; ++t) {
    const Task k = decode(g, t);
    if (k.phase == PH_NONE) continue;
    const uint64_t len = (k.hi - k.lo) * es;
    const uint64_t w = lines_for(g, len) * g.line_bytes;
    const int r = k.rank;
    switch (g.kind) {
      case K_COPY:
        b.rd += len; b.wr += len;
        break;
      case K_ONESHOT:
        if (!lines) {
          b.rd += n * len; b.wr += len; b.link[r] += (n - 1) * len;
        } else if (k.phase == PH_SEND) {
          b.rd += len; b.wr += w;
        } else {
          b.rd += (n - 1) * w + (g.in_place ? w : len); b.wr += len; b.link[r] += (n - 1) * len;
        }
        break;
      case K_TWOSHOT:
        if (!lines) {
          if (k.phase == PH_FOLD) { b.rd += n * len; b.wr += len; b.link[r] += (n - 1) * len; }
          else { b.rd += len; b.wr += len; b.link[r] += len; }
        } else if (k.phase == PH_SEND) {
          b.rd += len; b.wr += w;
        } else if (k.phase == PH_RECV_FOLD) {
          b.rd += len + (n - 1) * w; b.wr += len + w; b.link[r] += (n - 1) * len;
        } else {
          b.rd += w; b.wr += len; b.link[r] += len;
        }
        break;
      case K_RS_DIRECT:
        if (!lines) { b.rd += n * len; b.wr += len; b.link[r] += (n - 1) * len; }
        else if (k.phase == PH_SEND) { b.rd += len; b.wr += w; }
        else { b.rd += len + (n - 1) * w; b.wr += len; b.link[r] += (n - 1) * len; }
        break;
      case K_AG_DIRECT:
        if (!lines) { b.rd += len; b.wr += len; if (r != k.peer) b.link[r] += len; }
        else if (k.phase == PH_SEND) { b.rd += len; b.wr += w + len; }
        else { b.rd += w; b.wr += len; b.link[r] += len; }
        break;
      case K_RING: {
        const int s = k.step, last = g.steps - 1;
        if (!lines) {
          if (g.op == OP_ALLGATHER) {
            b.rd += len; b.wr += len;
            if (s > 0) b.link[r] += len;
          } else if (g.op == OP_ALLREDUCE && s >= n - 1) {
            b.rd += len; b.wr += len; b.link[r] += len;
          } else {
            b.rd += 2 * len; b.wr += len; b.link[r] += len;
          }
        } else if (s == 0) {
          b.rd += len; b.wr += w;
          if (g.op == OP_ALLGATHER) b.wr += len;  // rank j's own copy
        } else {
          const bool reduce = g.op != OP_ALLGATHER && s <= n - 1;
          b.rd += w + (reduce ? len : 0);
          b.link[r] += len;
          const bool keeps = !reduce || s == n - 1;  // writes its output buffer
          if (keeps) b.wr += len;
          if (s < last) b.wr += w;
          if (g.op == OP_REDUCE_SCATTER && s == last) {}  // last step: output only
        }
        break;
      }
      case K_TREE: {
        if (k.phase == PH_TREE_UP) {  // own input + each child's partial -> own output
          const uint64_t kids = (2 * k.peer + 1 < n) + (2 * k.peer + 2 < n);
          b.rd += (1 + kids) * len; b.wr += len; b.link[r] += kids * len;
        } else {                      // the parent's sum -> own output
          b.rd += len; b.wr += len; b.link[r] += len;
        }
        break;
      }
      default:
        break;
    }
  }
  return b;
}

}  // namespace ar
