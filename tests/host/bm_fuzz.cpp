// Randomised operation sequences against the C++ block manager, built for the
// host with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  Every call goes through the C ABI; after
// each one the pool-wide invariants are checked through the same ABI:
// referenced + free + evictable = all blocks, each sequence holds
// ceil(len / BS) blocks, refcounts equal table references, and a failed call
// leaves the free count, the stats and every table unchanged.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pa.h"

namespace pa {
pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  char buf[256];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace pa

#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);   \
      std::exit(2);                                                         \
    }                                                                       \
  } while (0)

struct State {
  std::vector<int64_t> stats;
  std::map<int64_t, std::vector<int32_t>> tables;
  int32_t free_blocks;
};

static std::vector<int32_t> table_of(pa_bm* bm, int64_t seq, int32_t bs) {
  const int32_t len = pa_bm_seq_len(bm, seq);
  const int32_t stride = len / bs + 2;
  std::vector<int32_t> tab(stride, -7);
  int32_t ctx = -1;
  CHECK(pa_bm_export(bm, &seq, 1, stride, tab.data(), &ctx) == PA_OK);
  CHECK(ctx == len);
  std::vector<int32_t> out;
  for (int32_t b : tab)
    if (b >= 0) out.push_back(b);
  CHECK(int64_t(out.size()) == (int64_t(len) + bs - 1) / bs);
  return out;
}

static State snapshot(pa_bm* bm, int32_t bs, const std::vector<int64_t>& live) {
  State s;
  s.stats.assign(5, 0);
  CHECK(pa_bm_stats(bm, s.stats.data()) == PA_OK);
  for (int64_t q : live) s.tables[q] = table_of(bm, q, bs);
  s.free_blocks = pa_bm_num_free(bm);
  return s;
}

static void invariants(pa_bm* bm, int32_t n, int32_t bs, const std::vector<int64_t>& live) {
  std::vector<int32_t> refs(n, 0);
  for (int64_t q : live)
    for (int32_t b : table_of(bm, q, bs)) {
      CHECK(b >= 0 && b < n);
      ++refs[b];
    }
  int32_t referenced = 0;
  for (int32_t b = 0; b < n; ++b) {
    CHECK(pa_bm_refcount(bm, b) == refs[b]);
    referenced += refs[b] > 0;
  }
  int64_t cs[4];
  CHECK(pa_bm_cache_stats(bm, cs) == PA_OK);
  // num_free counts the free stack and the evictable cached blocks
  CHECK(referenced + pa_bm_num_free(bm) == n);
  std::vector<int32_t> fl(n + 1);
  const int32_t nf = pa_bm_free_list(bm, fl.data(), n + 1);
  CHECK(nf + cs[1] == pa_bm_num_free(bm));
  for (int32_t i = 0; i < nf; ++i) CHECK(refs[fl[i]] == 0);
  CHECK(pa_bm_num_seqs(bm) == int32_t(live.size()));
}

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 200;
  std::mt19937_64 rng(12345);
  for (int r = 0; r < rounds; ++r) {
    const int32_t n = 8 + int32_t(rng() % 40);
    const int32_t bs = 1 << (rng() % 5);  // 1..16
    pa_bm* bm = pa_bm_create(n, bs, nullptr);
    CHECK(bm);
    std::vector<int64_t> live, swapped;
    std::vector<int32_t> buf(4096), buf2(4096);
    for (int op = 0; op < 300; ++op) {
      const int kind = int(rng() % 10);
      const int64_t seq = int64_t(rng() % 12);
      const int32_t len = int32_t(rng() % (3 * bs * 4 + 1));
      const State before = snapshot(bm, bs, live);
      pa_status st = PA_OK;
      bool is_live = false, is_swapped = false;
      for (int64_t q : live) is_live |= q == seq;
      for (int64_t q : swapped) is_swapped |= q == seq;
      switch (kind) {
        case 0: st = pa_bm_add_seq(bm, seq, len, buf.data()); if (!st) live.push_back(seq); break;
        case 1: st = pa_bm_admit(bm, seq, len, int32_t(rng() % 3), buf.data()); if (!st) live.push_back(seq); break;
        case 2: {
          std::vector<int32_t> tok(len);
          for (auto& t : tok) t = int32_t(rng() % 3);
          int32_t hit = -1;
          st = pa_bm_add_seq_cached(bm, seq, tok.data(), len, buf.data(), &hit);
          if (!st) {
            CHECK(hit >= 0 && hit % bs == 0 && (hit < len || len == 0));
            live.push_back(seq);
          }
          break;
        }
        case 3: {
          std::vector<int64_t> batch;
          for (int64_t q : live)
            if (rng() % 2) batch.push_back(q);
          int32_t ncow = -1;
          st = pa_bm_append_slots(bm, batch.data(), int32_t(batch.size()), buf.data(), buf2.data(), &ncow);
          if (!st) CHECK(ncow >= 0 && ncow <= int32_t(batch.size()));
          break;
        }
        case 4: {
          const int64_t child = int64_t(rng() % 12);
          st = pa_bm_fork(bm, seq, child);
          if (!st) live.push_back(child);
          break;
        }
        case 5:
          st = pa_bm_free_seq(bm, seq);
          if (!st) live.erase(std::find(live.begin(), live.end(), seq));
          break;
        case 6: {
          int32_t cnt = -1;
          st = pa_bm_swap_out(bm, seq, buf.data(), &cnt);
          if (!st) {
            live.erase(std::find(live.begin(), live.end(), seq));
            swapped.push_back(seq);
          }
          break;
        }
        case 7: {
          int32_t cnt = -1;
          st = pa_bm_swap_in(bm, seq, buf.data(), &cnt);
          if (!st) {
            swapped.erase(std::find(swapped.begin(), swapped.end(), seq));
            live.push_back(seq);
          }
          break;
        }
        case 8: {
          int64_t occ[4];
          CHECK(pa_bm_occupancy(bm, occ) == PA_OK);
          CHECK(occ[0] >= 0 && occ[1] >= 0 && occ[2] >= 0 && occ[3] >= 0);
          break;
        }
        default:
          if (rng() % 4 == 0) CHECK(pa_bm_cache_clear(bm) == PA_OK);
          break;
      }
      (void)is_live;
      (void)is_swapped;
      if (st != PA_OK) {
        // a failed call changes nothing
        const State after = snapshot(bm, bs, live);
        CHECK(after.stats == before.stats && after.tables == before.tables &&
              after.free_blocks == before.free_blocks);
      }
      invariants(bm, n, bs, live);
    }
    pa_bm_destroy(bm);
  }
  std::printf("ok %d rounds\n", rounds);
  return 0;
}
