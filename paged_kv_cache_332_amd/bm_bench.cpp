// Host cost of the block manager's calls, measured natively (no Python or
// ctypes in the timed loops).  Allocation in paged attention is meant to be
// fast and predictable (glossary "What is Paged Attention?": fixed-size
// blocks make allocation cheap); this prints, as one JSON line, the mean
// nanoseconds per call of each pa_bm_* operation a decode server issues, on
// shapes of the batch-64 grouped-query workload (64 sequences, block size 16,
// contexts of 128..4096 tokens, tables of 300 entries).
//
// Built next to libpa.so by build.py; run ./bm_bench [seconds per op].
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <random>
#include <string>
#include <vector>

#include "pa.h"

namespace {

using Clock = std::chrono::steady_clock;

// Mean ns per call of body(k) over batches of `batch` calls until `budget`
// seconds have passed; setup(k) runs untimed before each batch.
double time_op(double budget, int batch, const std::function<void(int)>& setup, const std::function<void(int)>& body,
               long long* calls_out) {
  double ns = 0;
  long long calls = 0;
  const auto t_end = Clock::now() + std::chrono::duration<double>(budget);
  for (int k = 0; Clock::now() < t_end; ++k) {
    setup(k);
    const auto t0 = Clock::now();
    for (int i = 0; i < batch; ++i) body(i);
    ns += std::chrono::duration<double, std::nano>(Clock::now() - t0).count();
    calls += batch;
  }
  *calls_out = calls;
  return calls ? ns / calls : 0;
}

void check(pa_status st, const char* what) {
  if (st != PA_OK) {
    std::fprintf(stderr, "%s failed: %s\n", what, pa_last_error());
    std::exit(1);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const double budget = argc > 1 ? std::atof(argv[1]) : 0.3;
  const int B = 64, BS = 16, stride = 300;  // room for 256 appended tokens
  std::mt19937 rng(12345);
  std::uniform_int_distribution<int> ctx_dist(128, 4096);
  std::vector<int32_t> ctx(B);
  for (auto& c : ctx) c = ctx_dist(rng);
  std::vector<int64_t> ids(B);
  for (int i = 0; i < B; ++i) ids[i] = i;
  std::string json = "{";
  auto add = [&](const char* name, double ns, long long calls, const std::string& unit) {
    char buf[320];
    std::snprintf(buf, sizeof buf, "%s\"%s\": {\"ns\": %.1f, \"calls\": %lld, \"per\": \"%s\"}", json.size() > 1 ? ", " : "",
                  name, ns, calls, unit.c_str());
    json += buf;
  };
  long long calls = 0;

  // decode step: append one token to each of 64 sequences, export their
  // tables, read their shared-prefix counts; the batch restarts from the
  // initial lengths every 256 steps
  const int32_t N = 200000;
  pa_bm* bm = pa_bm_create(N, BS, nullptr);
  std::vector<int32_t> slots(B), pairs(2 * B), tables(size_t(B) * stride), lens(B);
  int32_t ncow = 0;
  auto reset = [&] {
    for (int i = 0; i < B; ++i) {
      pa_bm_free_seq(bm, ids[i]);
      check(pa_bm_add_seq(bm, ids[i], ctx[i], nullptr), "add_seq");
    }
  };
  for (int i = 0; i < B; ++i) check(pa_bm_add_seq(bm, ids[i], ctx[i], nullptr), "add_seq");
  double ns = time_op(budget, 256, [&](int) { reset(); },
                      [&](int) { check(pa_bm_append_slots(bm, ids.data(), B, slots.data(), pairs.data(), &ncow), "append"); },
                      &calls);
  add("append_slots_64", ns, calls, "call of 64 sequences");
  ns = time_op(budget, 256, [&](int) {},
               [&](int) { check(pa_bm_export(bm, ids.data(), B, stride, tables.data(), lens.data()), "export"); }, &calls);
  add("export_64", ns, calls, "call of 64 sequences");
  volatile int32_t sink = 0;
  ns = time_op(budget, 4096, [&](int) {}, [&](int i) { sink = sink + pa_bm_shared_blocks(bm, ids[i % B]); }, &calls);
  add("shared_blocks", ns, calls, "sequence");

  // a sequence's whole life at the mean context: add (133 blocks), free
  const int64_t extra = 1000;
  ns = time_op(budget, 1, [&](int) {}, [&](int) { check(pa_bm_add_seq(bm, extra, 2112, nullptr), "add"); pa_bm_free_seq(bm, extra); },
               &calls);
  double both = ns;
  ns = time_op(budget, 1, [&](int) { pa_bm_free_seq(bm, extra); },
               [&](int) { check(pa_bm_add_seq(bm, extra, 2112, nullptr), "add"); }, &calls);
  add("add_seq_2112", ns, calls, "call (133 blocks)");
  add("free_seq_2112", both - ns, calls, "call (133 blocks), from add+free minus add");
  pa_bm_free_seq(bm, extra);

  // admission with headroom of a 512-token prompt (succeeds), then release
  ns = time_op(budget, 1, [&](int) { pa_bm_free_seq(bm, extra); },
               [&](int) { check(pa_bm_admit(bm, extra, 512, 64, nullptr), "admit"); }, &calls);
  add("admit_512", ns, calls, "call (32 blocks)");
  pa_bm_free_seq(bm, extra);

  // fork of a 2048-token parent (128 shared blocks) and the child's release
  check(pa_bm_add_seq(bm, 2000, 2048, nullptr), "parent");
  ns = time_op(budget, 1, [&](int) { pa_bm_free_seq(bm, 2001); }, [&](int) { check(pa_bm_fork(bm, 2000, 2001), "fork"); },
               &calls);
  add("fork_2048", ns, calls, "call (128 blocks)");
  pa_bm_free_seq(bm, 2001);
  pa_bm_free_seq(bm, 2000);

  // a prompt of 2048 shared + 256 own tokens whose prefix is cached
  std::vector<int32_t> prompt(2304);
  for (int t = 0; t < 2304; ++t) prompt[t] = t < 2048 ? t * 7 + 1 : int32_t(rng() % 32000);
  int32_t cached = 0;
  check(pa_bm_add_seq_cached(bm, 3000, prompt.data(), 2048 + 16, nullptr, &cached), "cache the prefix");
  ns = time_op(budget, 1, [&](int) { pa_bm_free_seq(bm, 3001); },
               [&](int) { check(pa_bm_add_seq_cached(bm, 3001, prompt.data(), 2304, nullptr, &cached), "cached"); }, &calls);
  add("add_seq_cached_2304", ns, calls,
      "call (" + std::to_string(cached) + " cached tokens reused, " + std::to_string(2304 - cached) + " new)");
  pa_bm_free_seq(bm, 3001);
  pa_bm_free_seq(bm, 3000);

  // the stream kernel's split for the decode step (64 sequences, 8 kv
  // heads, 256 workgroups)
  std::vector<int32_t> pre(B + 1, 0);
  for (int i = 0; i < B; ++i) pre[i + 1] = pre[i] + (ctx[i] + 15) / 16;
  std::vector<int32_t> plan(8 * 1024 + 8 * B * 8 + 64);
  int32_t ncut = 0;
  ns = time_op(budget, 256, [&](int) {},
               [&](int) { sink = sink + int32_t(pa_stream_plan(pre.data(), B, 8, 256, nullptr, plan.data(), plan.size(), &ncut)); },
               &calls);
  add("stream_plan_64x8_grid256", ns, calls, "call");
  pa_bm_destroy(bm);
  json += "}";
  std::printf("%s\n", json.c_str());
  return 0;
}
