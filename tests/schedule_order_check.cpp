// Host check of the ticket order of every schedule (compiled and run by
// tests/test_schedule_order.py).  The kernels are deadlock-free only if every
// task a task waits on has a smaller ticket; this walks decode() over every
// ticket of many geometries and checks that, and that every task of the
// schedule appears exactly once.
#include <cstdio>
#include <map>
#include <set>
#include <tuple>

#include "../all_reduce_reduction_rank_amd/csrc/plan.hpp"

using namespace ar;

static int fail(const char* what, int op, int algo, int proto, int n, unsigned long long count, unsigned long long t) {
  std::printf("FAIL %s: op %d algo %d proto %d n %d count %llu ticket %llu\n", what, op, algo, proto, n, count, t);
  return 1;
}

static int check(int op, int algo, int proto, int dt, int n, uint64_t count, uint64_t chunk, int in_place) {
  Geometry g;
  if (!make_geometry(op, algo, proto, dt, n, count, chunk, in_place, &g)) return 0;  // unsupported combination
  if (g.kind == K_COPY) return 0;
  std::set<std::tuple<int, uint64_t, uint64_t, int, int>> done;  // (phase, block, tile, rank/pos, step)
  std::map<std::pair<uint64_t, int>, uint64_t> ring;            // (chain, step) -> ticket
  for (uint64_t t = 0; t < g.ntasks; ++t) {
    const Task k = decode(g, t);
    if (k.phase == PH_NONE) continue;
    if (g.kind == K_RING) {
      if (ring.count({k.chain, k.step})) return fail("ring duplicate", op, algo, proto, n, count, t);
      if (k.step > 0 && !ring.count({k.chain, k.step - 1})) return fail("ring order", op, algo, proto, n, count, t);
      ring[{k.chain, k.step}] = t;
    } else if (g.kind == K_TREE) {
      const auto key = std::make_tuple(k.phase, k.block, k.tile, k.peer, 0);
      if (done.count(key)) return fail("tree duplicate", op, algo, proto, n, count, t);
      const int p = k.peer;
      if (k.phase == PH_TREE_UP) {
        for (int c : {2 * p + 1, 2 * p + 2})
          if (c < n && !done.count(std::make_tuple((int)PH_TREE_UP, k.block, k.tile, c, 0)))
            return fail("tree up order", op, algo, proto, n, count, t);
      } else {
        const int parent = (p - 1) / 2;
        const int ph = parent == 0 ? PH_TREE_UP : PH_TREE_DOWN;
        if (!done.count(std::make_tuple(ph, k.block, k.tile, parent, 0)))
          return fail("tree down order", op, algo, proto, n, count, t);
      }
      done.insert(key);
    } else if (g.kind == K_TWOSHOT && proto == PROTO_SIMPLE) {
      if (k.phase == PH_FOLD) done.insert(std::make_tuple(0, k.block, k.tile, 0, 0));
      else if (!done.count(std::make_tuple(0, k.block, k.tile, 0, 0))) return fail("two-shot order", op, algo, proto, n, count, t);
    } else if (proto != PROTO_SIMPLE) {  // phased line schedules: receivers after every sender
      if (k.phase == PH_SEND) {
        done.insert(std::make_tuple((int)PH_SEND, k.block, k.tile, k.rank, 0));
      } else if (k.phase == PH_RECV_FOLD) {
        for (int i = 0; i < n; ++i) {
          if (g.kind == K_ONESHOT) {
            if ((i != k.rank || in_place) && !done.count(std::make_tuple((int)PH_SEND, (uint64_t)0, k.tile, i, 0)))
              return fail("one-shot line order", op, algo, proto, n, count, t);
          } else if (i != (int)k.block && !done.count(std::make_tuple((int)PH_SEND, k.block, k.tile, i, 0))) {
            return fail("direct line order", op, algo, proto, n, count, t);
          }
        }
        done.insert(std::make_tuple((int)PH_RECV_FOLD, k.block, k.tile, 0, 0));
      } else if (k.phase == PH_RECV_COPY) {
        if (g.kind == K_TWOSHOT && !done.count(std::make_tuple((int)PH_RECV_FOLD, k.block, k.tile, 0, 0)))
          return fail("two-shot line gather order", op, algo, proto, n, count, t);
        if (g.kind == K_AG_DIRECT && !done.count(std::make_tuple((int)PH_SEND, k.block, k.tile, (int)k.block, 0)))
          return fail("all-gather line order", op, algo, proto, n, count, t);
      }
    }
  }
  return 0;
}

int main() {
  int bad = 0, cases = 0;
  const uint64_t counts[] = {1, 7, 1000, 70001, 1 << 20, 6553600, 67108864 / 4};
  const uint64_t chunks[] = {0, 16, 240, 4096, 524288};
  for (int op = 0; op < 3; ++op)
    for (int algo = 0; algo < 4; ++algo)
      for (int proto = 0; proto < 3; ++proto)
        for (int n : {2, 3, 5, 8})
          for (uint64_t c : counts)
            for (uint64_t ch : chunks) {
              if (ch && algo != ALGO_RING) continue;
              // keep the run short: tiny chunks only on small buffers, large
              // buffers with Simple and the default chunk only
              if (ch && ch < 4096 && c > 70001) continue;
              if (c > (1u << 20) && (ch || proto != PROTO_SIMPLE)) continue;
              for (int ip = 0; ip < (op == 0 ? 2 : 1); ++ip) {
                ++cases;
                bad += check(op, algo, proto, DT_F32, n, c, ch, ip);
                if (bad > 5) return 1;
              }
            }
  std::printf("checked %d geometries, %d bad\n", cases, bad);
  return bad ? 1 : 0;
}
