// Host check of a communicator's call log (compiled and run by
// tests/test_call_log.py): the last CAP calls are kept, handed out oldest
// first with their sequence numbers, and formatted on one line.
#include <cstdio>
#include <cstring>

#include "../all_reduce_reduction_rank_amd/csrc/calllog.hpp"

using namespace ar;

static int bad = 0;
#define CHECK(c)                                        \
  do {                                                  \
    if (!(c)) {                                         \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);  \
      ++bad;                                            \
    }                                                   \
  } while (0)

static ar_call_record rec(uint64_t count) {
  ar_call_record r = {};
  r.op = 0; r.algo = 2; r.proto = 0; r.dtype = 0; r.nranks = 8;
  r.grid = 768; r.batch = 2; r.count = count; r.ntasks = 10 * count; r.tile_bytes = 32768;
  return r;
}

int main() {
  CallLog log;
  ar_call_record out[CallLog::CAP];
  CHECK(log.copy(out, CallLog::CAP) == 0);
  for (uint64_t i = 1; i <= 3; ++i) log.add(rec(100 * i));
  CHECK(log.copy(out, CallLog::CAP) == 3);
  for (int i = 0; i < 3; ++i) CHECK(out[i].seq == (uint64_t)i + 1 && out[i].count == 100ull * (i + 1));
  CHECK(log.copy(out, 2) == 2);  // the two most recent, oldest first
  CHECK(out[0].seq == 2 && out[1].seq == 3);
  for (uint64_t i = 4; i <= 40; ++i) log.add(rec(100 * i));
  CHECK(log.copy(out, CallLog::CAP) == CallLog::CAP);
  for (int i = 0; i < CallLog::CAP; ++i) CHECK(out[i].seq == 40 - CallLog::CAP + 1 + (uint64_t)i);
  CHECK(out[CallLog::CAP - 1].count == 4000);
  CHECK(log.copy(out, -1) == 0);
  char line[320];
  format_record(line, sizeof(line), out[CallLog::CAP - 1]);
  CHECK(std::strcmp(line, "call 40: allreduce ring/simple f32 N=8 count=4000 out of place, tile 32768 B, "
                          "40000 tasks, grid 768 x batch 2") == 0);
  std::printf("%s\n%d bad\n", line, bad);
  return bad ? 1 : 0;
}
