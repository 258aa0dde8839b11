// Host check of the tile choice of the schedules whose tasks never wait
// (Simple one-shot out of place, direct reduce-scatter and all-gather),
// compiled and run by tests/test_tile_rule.py.  Such a call launches without
// the ticket counter when one grid covers all its tasks; the planner grows
// the tile toward that (FIXED_GRID_TASKS tasks) within a per-schedule bound.
// For many shapes this checks: a call fits the grid whenever a tile within
// the bound would let it; no tile exceeds its bound or shrinks below the
// size-based choice; tiles stay whole 16-byte vectors.
#include <cstdio>
#include <initializer_list>
#include <vector>

#include "../all_reduce_reduction_rank_amd/csrc/plan.hpp"

using namespace ar;

int main() {
  const int ops[] = {OP_ALLREDUCE, OP_REDUCE_SCATTER, OP_ALLGATHER};
  const int dts[] = {DT_F32, DT_BF16, DT_I32};
  int bad = 0, checked = 0, grown = 0;
  for (int op : ops)
    for (int dt : dts)
      for (int n = 2; n <= MAX_RANKS; ++n)
        for (uint64_t kib = 1; kib <= (1u << 20); kib *= 2)
          for (uint64_t extra : {0ull, 1ull, 3ull}) {  // whole and ragged sizes
            const uint64_t es = (uint64_t)esize_of(dt);
            const uint64_t bytes = kib * 1024 + extra * 2 * es * 5;
            const uint64_t count = op == OP_ALLREDUCE ? bytes / es : bytes / es / n;
            if (count == 0) continue;
            Geometry g;
            if (!make_geometry(op, ALGO_ONESHOT, PROTO_SIMPLE, dt, n, count, 0, 0, &g)) continue;
            ++checked;
            const uint64_t rank_bytes = g.total * es;
            const uint64_t tile_b = g.tile * es;
            const uint64_t base = pick_tile_bytes(PROTO_SIMPLE, rank_bytes, g.kind, false, n);
            // one-shot: 128 KiB tiles when the N inputs exceed one die's 4 MiB L2
            // (the tile's N programs then run on one die), else 16 KiB
            const uint64_t oneshot_bound = (uint64_t)n * rank_bytes > (4ull << 20) ? 131072 : 16384;
            const uint64_t bound = g.kind == K_ONESHOT ? oneshot_bound : g.kind == K_RS_DIRECT ? 65536
                                                       : simple_tile_cap(rank_bytes, g.kind, false);
            const uint64_t per_row = g.kind == K_AG_DIRECT ? (uint64_t)n * n : (uint64_t)n;
            const uint64_t extent_b = (g.kind == K_ONESHOT ? g.total : g.block) * es;
            // the smallest tile (whole vectors) that fits the grid
            const uint64_t rows = FIXED_GRID_TASKS / per_row;
            const uint64_t need = cdiv(cdiv(extent_b, rows), 16) * 16;
            const bool fits = g.ntasks <= FIXED_GRID_TASKS;
            if (tile_b % 16 || tile_b < base || (tile_b > base && tile_b > bound) ||
                (need <= bound && !fits) || (tile_b > base && tile_b != need)) {
              std::printf("FAIL op %d dt %d n %d bytes %llu: tile %llu base %llu bound %llu need %llu tasks %llu\n",
                          op, dt, n, (unsigned long long)bytes, (unsigned long long)tile_b,
                          (unsigned long long)base, (unsigned long long)bound, (unsigned long long)need,
                          (unsigned long long)g.ntasks);
              ++bad;
            }
            if (tile_b > base) ++grown;
          }
  // die_ticket: over a grid of XCDS * G * ceil(groups / XCDS) workgroups,
  // every ticket of `groups` groups of G appears exactly once, all G tickets
  // of a group on one die (workgroup b on die b % XCDS), and the workgroups
  // left over get tickets past the last.
  int placed = 0;
  for (uint32_t G = 1; G <= (uint32_t)MAX_RANKS; ++G)
    for (uint32_t groups = 1; groups <= 70; ++groups) {
      const uint32_t grid = (uint32_t)(XCDS * G * cdiv(groups, XCDS));
      const uint32_t ntasks = groups * G;
      std::vector<int> seen(ntasks, 0), die(groups, -1);
      for (uint32_t b = 0; b < grid; ++b) {
        const uint64_t t = die_ticket(b, G);
        if (t >= ntasks) continue;
        ++seen[t];
        const int d = (int)(b % XCDS), m = (int)(t / G);
        if (die[m] < 0) die[m] = d;
        if (die[m] != d) { std::printf("FAIL die_ticket G %u groups %u: group %d on two dies\n", G, groups, m); ++bad; }
      }
      for (uint32_t t = 0; t < ntasks; ++t)
        if (seen[t] != 1) { std::printf("FAIL die_ticket G %u groups %u: ticket %u seen %d times\n", G, groups, t, seen[t]); ++bad; }
      ++placed;
    }
  std::printf("%d shapes, %d grown, %d placements, %d bad\n", checked, grown, placed, bad);
  return bad ? 1 : 0;
}
