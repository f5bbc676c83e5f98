// One decode step of a batch in native code: the host block manager hands
// every sequence the slot of its new token (taking a block when the last one
// is full, copying a shared last block first), the step's bookkeeping goes to
// the device in one copy, and the kernels run in order on one stream.  A
// request fills the block it holds before it takes another and copies a block
// it shares before it writes to it ("Paged Attention: Virtual Memory for the
// KV Cache", §The fix borrowed from operating systems, §Sharing comes almost
// for free); the attention then follows the block tables (glossary "What is
// Paged Attention?").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <vector>

#include "pa_internal.h"
#include "pa_kernels.h"

namespace {

// Device-visible address of `p`: pinned host memory maps to its device
// address (the same on a unified address space), device memory to itself
// when `allow_device`; anything else gives nullptr.  The last few lookups are
// cached: callers rotate a handful of step records.
int32_t* device_view(const int32_t* p, bool allow_device) {
  struct Entry {
    const void* p;
    void* dev;
    bool device;
  };
  static thread_local Entry cache[16] = {};
  static thread_local int next = 0;
  for (const Entry& e : cache)
    if (e.p == p) return (e.device && !allow_device) ? nullptr : static_cast<int32_t*>(e.dev);
  hipPointerAttribute_t attr{};
  void* dev = nullptr;
  bool device = false;
  if (hipPointerGetAttributes(&attr, p) == hipSuccess) {
    if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
      dev = attr.devicePointer;
    } else if (attr.type == hipMemoryTypeDevice) {
      dev = const_cast<int32_t*>(p);
      device = true;
    }
  }
  (void)hipGetLastError();  // a plain host pointer leaves an error behind
  cache[next] = Entry{p, dev, device};
  next = (next + 1) % 16;
  return (device && !allow_device) ? nullptr : static_cast<int32_t*>(dev);
}

constexpr size_t kHeaderWords = 4;

// floor(num / den) for 0 <= num < 2^62, den > 0: the quotient in double
// precision is within a few units of the exact one (num may exceed 2^53), and
// exact 64-bit products correct it (a hardware 64-bit division costs tens of
// cycles, and a plan takes one per workgroup).
inline int64_t floor_div(int64_t num, int64_t den) {
  int64_t q = static_cast<int64_t>(static_cast<double>(num) / static_cast<double>(den));
  while (q > 0 && q * den > num) --q;
  while ((q + 1) * den <= num) ++q;
  return q;
}

// Word where the cut-item entries start in a plan for `grid` workgroups
// (after the 4 grid + 1 wave starts, rounded up to 4 words).
size_t plan_entries(int64_t grid) { return size_t(4 * grid + 1 + 3) / 4 * 4; }

// Words of a step record for n sequences: the bookkeeping, the tile prefix
// sums and room for the stream kernel's plan with `grid` workgroups.
size_t record_words(int64_t n, int64_t stride, int64_t hkv, int64_t grid) {
  // (the plan: wave starts padded to 4 words, an 8-word entry per cut item,
  // at most two cut items per wave in the full wave list)
  const size_t w = size_t(n) * (6 + stride + 8 * hkv) + 1 + kHeaderWords + 3 + (grid ? 12 * grid + 4 : 0);
  return (w + 3) / 4 * 4;
}

// Where the parts of a record for n sequences start: slots [n], copy-on-write
// pairs [n][2], lengths [n], tables [n][stride], tile prefix sums [n + 1],
// shared leading blocks [n], header, plan.  The header holds the
// copy-on-write pair count, the stream grid the plan was made for (0: no
// plan), the cut-item count and the words in use.
struct Layout {
  size_t pre, shared, header, plan;
};
Layout layout(int64_t n, int64_t stride) {
  Layout l;
  l.pre = size_t(4 * n + n * stride);
  l.shared = l.pre + size_t(n) + 1;
  l.header = l.shared + size_t(n);
  l.plan = (l.header + kHeaderWords + 3) / 4 * 4;  // 16-byte aligned, as are the entries
  return l;
}

// The device part of a step (or of another layer's step on the same record):
// phases bit 0 = copy-on-write copies and the KV write, bit 1 = the decode
// pass, bit 2 = the merge.  With `stage`, bit 0 also copies the record from
// its host view to stage_dev in the same launch as the KV write.
pa_status run_device(const char* fn, const int32_t* stage_host, const int32_t* host_view, int32_t* stage_dev,
                     int32_t n, int32_t table_stride, bool stage, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const void* q, void* out, pa_dtype out_dtype, pa_dtype kv_dtype,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                     pa_kernel kernel, void* stream, int phases, void* pass_begin, void* pass_end,
                     int32_t* d_times) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Layout lo = layout(n, table_stride);
  const int32_t* hdr = stage_host + lo.header;
  const int32_t ncow = hdr[0], grid = hdr[1], ncut = hdr[2];
  const size_t words = (size_t(hdr[3]) + 3) / 4 * 4;
  int32_t max_ctx = 0;
  for (int32_t i = 0; i < n; ++i) max_ctx = std::max(max_ctx, stage_host[3 * n + i]);
  if (phases & 1) {
    if (!k_new || !v_new || (reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15u)
      return pa::fail(PA_ERR_INVALID, "%s: k_new and v_new must be 16-byte aligned device memory", fn);
    if (stage && host_view) {
      // the kernels read the record where the host wrote it: copy-on-write
      // copies, then one launch that copies the record to the device and
      // writes the new tokens' keys and values
      if (ncow) {
        if (pa_status st = pa_copy_blocks(k_cache, v_cache, host_view + n, ncow, num_kv_heads, head_dim, block_size,
                                          num_blocks, kv_dtype, stream))
          return st;
      }
      if (pa_status st = pa_write_kv(k_cache, v_cache, k_new, v_new, stage_dev, 0, num_kv_heads, head_dim,
                                     block_size, num_blocks, kv_dtype, stream))
        return st;  // validates the cache arguments; writes nothing
      if (hipError_t e = pa::launch_step_stage(host_view, stage_dev, static_cast<int64_t>(words), n, k_cache,
                                               v_cache, k_new, v_new, num_kv_heads, head_dim, block_size,
                                               kv_dtype == PA_F32 ? 4 : 2, stage_host, s))
        return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    } else {
      if (stage) {
        if (hipError_t e = hipMemcpyAsync(stage_dev, stage_host, words * sizeof(int32_t), hipMemcpyHostToDevice, s))
          return pa::fail(PA_ERR_HIP, "%s: copy of the step record: %s", fn, hipGetErrorString(e));
      }
      if (ncow) {
        if (pa_status st = pa_copy_blocks(k_cache, v_cache, stage_dev + n, ncow, num_kv_heads, head_dim, block_size,
                                          num_blocks, kv_dtype, stream))
          return st;
      }
      if (pa_status st = pa_write_kv(k_cache, v_cache, k_new, v_new, stage_dev, n, num_kv_heads, head_dim,
                                     block_size, num_blocks, kv_dtype, stream))
        return st;
    }
  }
  const int32_t* d_ctx = stage_dev + 3 * n;
  const int32_t* d_tables = stage_dev + 4 * n;
  pa::StreamExtras ex{stage_dev + lo.pre, nullptr, nullptr, nullptr, 0, d_times, stage_dev + lo.shared};
  if (grid > 0) {
    const int32_t* plan = stage_dev + lo.plan;
    ex.wave_start = plan;
    ex.cut_entry = plan + plan_entries(grid);
    ex.cut_workers = ex.cut_entry + 8 * int64_t(ncut);
    ex.num_cut = ncut;
  }
  if (phases & 2) {
    if (pass_begin) {
      if (hipError_t e = hipEventRecord(static_cast<hipEvent_t>(pass_begin), s))
        return pa::fail(PA_ERR_HIP, "%s: event: %s", fn, hipGetErrorString(e));
    }
    if (pa_status st = pa::decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, d_tables, table_stride, d_ctx,
                                       max_ctx, n, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                                       partition_size, workspace, workspace_bytes, stream, kernel, PA_PHASE_PASS,
                                       &ex))
      return st;
    if (pass_end) {
      if (hipError_t e = hipEventRecord(static_cast<hipEvent_t>(pass_end), s))
        return pa::fail(PA_ERR_HIP, "%s: event: %s", fn, hipGetErrorString(e));
    }
  }
  if (phases & 4)
    return pa::decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, d_tables, table_stride, d_ctx, max_ctx, n,
                           num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                           workspace, workspace_bytes, stream, kernel, PA_PHASE_MERGE, &ex);
  return PA_OK;
}

// The stream kernel's split, planned on the host and written at `out`:
//   wave starts [4 grid + 1]: workgroup b takes tiles [T P_b / P, T P_(b+1) / P)
//     of the T = Hkv * pre[n] tiles (P_b the sum of the weights before it,
//     P their total), split evenly over its four waves;
//   then, from word plan_entries(grid) on (a multiple of 4), one 8-word entry
//     per item whose tiles fall to more than one wave: {2 * (seq * Hkv +
//     kvh) + (1 when the first wave holding the item started before it), the
//     number of those waves (non-empty ones only), the offset of the first in
//     the wave list, the first four of them (0 past the count), 0};
//   the wave list: every cut item's waves in order.
// Returns the words written; sets *ncut_out.
size_t build_plan(int32_t* out, const int32_t* pre, int32_t n, int32_t hkv, int32_t grid, const int32_t* weights,
                  int32_t* ncut_out) {
  const int64_t total = int64_t(hkv) * pre[n];
  const int64_t nw = int64_t(grid) * 4;
  int32_t* S = out;
  // (per-thread scratch, bound once: each use of a thread_local object in a
  // shared library can cost a call to look up its address)
  static thread_local std::vector<int64_t> wts_tls;
  static thread_local std::vector<int32_t> waves_tls;
  std::vector<int64_t>& wts = wts_tls;
  std::vector<int32_t>& waves = waves_tls;
  wts.resize(size_t(grid));
  int64_t all = 0;
  for (int32_t b = 0; b < grid; ++b) {
    wts[b] = weights ? std::clamp<int64_t>(weights[b], 1, 1 << 16) : 1;
    all += wts[b];
  }
  // workgroup b starts at floor(total * (weights before b) / all); each
  // boundary is computed once and ends one workgroup and starts the next
  int64_t before = 0, a0 = 0;
  for (int32_t b = 0; b < grid; ++b) {
    before += wts[b];
    const int64_t a1 = floor_div(total * before, all);
    for (int k = 0; k < 4; ++k) S[4 * b + k] = static_cast<int32_t>(a0 + (((a1 - a0) * k) >> 2));
    a0 = a1;
  }
  S[nw] = static_cast<int32_t>(total);
  // items in tile order, with the wave holding their first and last tile;
  // entries go straight to their place, the waves they list to scratch
  // (every cut item lists its waves, adjacent items share one: at most
  // nw + items in all)
  const size_t at = plan_entries(grid);
  std::fill(out + nw + 1, out + at, 0);
  int32_t* ent = out + at;
  waves.resize(size_t(nw) + size_t(n) * hkv + 1);
  int32_t* wl = waves.data();
  size_t nwl = 0, ncut = 0;
  int64_t w = 0;  // the last wave starting at or before the current tile
  for (int32_t s = 0; s < n; ++s) {
    const int64_t nt = pre[s + 1] - pre[s];
    if (nt == 0) continue;
    for (int32_t h = 0; h < hkv; ++h) {
      const int64_t gs = int64_t(hkv) * pre[s] + h * nt;
      while (w + 1 < nw && S[w + 1] <= gs) ++w;
      int64_t wh = w;
      while (wh + 1 < nw && S[wh + 1] <= gs + nt - 1) ++wh;
      if (wh != w) {
        const size_t off = nwl;
        for (int64_t x = w; x <= wh; ++x) {  // non-empty waves only
          wl[nwl] = static_cast<int32_t>(x);
          nwl += S[x] < S[x + 1];
        }
        const int32_t cnt = static_cast<int32_t>(nwl - off);
        int32_t* e = ent + 8 * ncut;
        e[0] = static_cast<int32_t>(2 * (int64_t(s) * hkv + h) + (S[w] < gs ? 1 : 0));
        e[1] = cnt;
        e[2] = static_cast<int32_t>(off);
        e[3] = wl[off];
        e[4] = cnt > 1 ? wl[off + 1] : 0;
        e[5] = cnt > 2 ? wl[off + 2] : 0;
        e[6] = cnt > 3 ? wl[off + 3] : 0;
        e[7] = 0;
        ++ncut;
      }
      w = wh;
    }
  }
  std::copy(wl, wl + nwl, ent + 8 * ncut);
  *ncut_out = static_cast<int32_t>(ncut);
  return at + 8 * ncut + nwl;
}

}  // namespace

extern "C" {

int64_t pa_stream_plan(const int32_t* tile_prefix, int32_t n, int32_t num_kv_heads, int32_t grid,
                       const int32_t* weights, int32_t* out, size_t out_words, int32_t* num_cut) {
  if (!tile_prefix || !out || !num_cut || n < 0 || num_kv_heads <= 0 || grid <= 0 || grid > pa::kStreamMaxGrid)
    return -1;
  if (tile_prefix[0] != 0) return -1;
  for (int32_t i = 0; i < n; ++i)
    if (tile_prefix[i + 1] < tile_prefix[i]) return -1;
  if (int64_t(num_kv_heads) * tile_prefix[n] >= (int64_t(1) << 31)) return -1;
  if (out_words < plan_entries(grid) + 8 * size_t(n) * num_kv_heads + 8 * size_t(grid)) return -1;
  return static_cast<int64_t>(build_plan(out, tile_prefix, n, num_kv_heads, grid, weights, num_cut));
}

pa_status pa_stream_class_finish(const int32_t* wave_times, int32_t grid, int32_t classes, double* out) {
  if (!wave_times || !out || grid <= 0 || classes <= 0)
    return pa::fail(PA_ERR_INVALID, "pa_stream_class_finish: bad arguments");
  const int32_t t0 = wave_times[0];
  int32_t first = 0;  // earliest start, relative to the first wave's
  for (int32_t i = 0; i < 4 * grid; ++i)
    first = std::min(first, static_cast<int32_t>(static_cast<uint32_t>(wave_times[2 * i]) - static_cast<uint32_t>(t0)));
  std::fill(out, out + classes, 0.0);
  static thread_local std::vector<int32_t> count_tls;
  std::vector<int32_t>& count = count_tls;
  count.assign(size_t(classes), 0);
  for (int32_t b = 0; b < grid; ++b) {
    int32_t end = INT32_MIN;
    for (int k = 0; k < 4; ++k)
      end = std::max(end, static_cast<int32_t>(static_cast<uint32_t>(wave_times[2 * (4 * b + k) + 1]) -
                                               static_cast<uint32_t>(t0)));
    out[b % classes] += double(int64_t(end) - first);
    ++count[b % classes];
  }
  for (int32_t c = 0; c < classes; ++c) out[c] = count[c] ? out[c] / count[c] : 0.0;
  return PA_OK;
}

size_t pa_step_record_words(int32_t max_seqs, int32_t table_stride, int32_t num_kv_heads) {
  if (max_seqs <= 0 || table_stride <= 0 || num_kv_heads <= 0) return 0;
  return record_words(max_seqs, table_stride, num_kv_heads, pa::kStreamMaxGrid);
}

pa_status pa_step(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* stage_host, int32_t* stage_dev,
                  size_t stage_words, int32_t table_stride, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  const void* q, void* out, pa_dtype out_dtype, pa_dtype kv_dtype, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                  int32_t partition_size, void* workspace, size_t workspace_bytes, pa_kernel kernel,
                  void* stream, void* pass_begin, void* pass_end, int32_t* max_ctx_out,
                  const int32_t* wg_weights, int32_t num_weights, int32_t* wave_times) {
  const char* fn = "pa_step";
  if (!bm || !seqs || !stage_host || !stage_dev || n <= 0 || table_stride <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_INVALID, "%s: bad arguments", fn);
  // every sequence must still fit the table stride after its new token, so
  // that the export below cannot fail once the manager has changed
  int32_t max_len = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t len = pa_bm_seq_len(bm, seqs[i]);
    if (len < 0) return pa::fail(PA_ERR_INVALID, "%s: unknown sequence %lld", fn, static_cast<long long>(seqs[i]));
    if (static_cast<int64_t>(len) + 1 > static_cast<int64_t>(table_stride) * block_size)
      return pa::fail(PA_ERR_INVALID, "%s: sequence %lld outgrows the table stride %d", fn,
                      static_cast<long long>(seqs[i]), table_stride);
    max_len = std::max(max_len, len + 1);
  }
  // the decode arguments, checked before anything changes
  if (pa_status st = pa::decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, stage_dev, table_stride,
                                     stage_dev, max_len, n, num_q_heads, num_kv_heads, head_dim, block_size,
                                     num_blocks, scale, partition_size, workspace, workspace_bytes, stream, kernel, 0,
                                     nullptr))
    return st;
  const int32_t grid = pa::stream_grid_selected(kernel, kv_dtype, n, num_q_heads, num_kv_heads, head_dim);
  if (stage_words < record_words(n, table_stride, num_kv_heads, grid))
    return pa::fail(PA_ERR_INVALID, "%s: the step record needs %zu words, %zu given", fn,
                    record_words(n, table_stride, num_kv_heads, grid), stage_words);
  if (wg_weights && num_weights != grid)
    return pa::fail(PA_ERR_INVALID, "%s: %d workgroup weights given, the stream kernel runs %d", fn, num_weights,
                    grid);
  // the new tokens' rows, checked here too: nothing below may fail once the
  // manager has changed
  if (!k_new || !v_new || (reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15u)
    return pa::fail(PA_ERR_INVALID, "%s: k_new and v_new must be 16-byte aligned device memory", fn);
  int32_t* d_times = nullptr;
  if (wave_times && !(d_times = device_view(wave_times, true)))
    return pa::fail(PA_ERR_INVALID, "%s: wave_times is neither pinned host nor device memory", fn);
  int32_t* slots = stage_host;
  int32_t* pairs = stage_host + n;
  int32_t* ctx = stage_host + 3 * n;
  int32_t* tables = stage_host + 4 * n;
  int32_t ncow = 0;
  if (pa_status st = pa_bm_append_slots(bm, seqs, n, slots, pairs, &ncow)) return st;
  if (pa_status st = pa_bm_export(bm, seqs, n, table_stride, tables, ctx)) return st;
  int32_t max_ctx = 0;
  for (int32_t i = 0; i < n; ++i) max_ctx = std::max(max_ctx, ctx[i]);
  if (max_ctx_out) *max_ctx_out = max_ctx;
  // tile (16-token) prefix sums, the header and the stream kernel's plan
  // follow the tables
  const Layout lo = layout(n, table_stride);
  int32_t* pre = stage_host + lo.pre;
  pre[0] = 0;
  for (int32_t i = 0; i < n; ++i) pre[i + 1] = pre[i] + (ctx[i] + 15) / 16;
  // blocks at the front of each table that other sequences also hold (a
  // forked or cached prefix): the pass reads them more than once, so their
  // loads keep the caching policy
  int32_t* shared = stage_host + lo.shared;
  for (int32_t i = 0; i < n; ++i) shared[i] = pa_bm_shared_blocks(bm, seqs[i]);
  int32_t ncut = 0;
  const bool planned = grid > 0 && int64_t(num_kv_heads) * pre[n] < (int64_t(1) << 31);
  const size_t plan_words =
      planned ? build_plan(stage_host + lo.plan, pre, n, num_kv_heads, grid, wg_weights, &ncut) : 0;
  int32_t* hdr = stage_host + lo.header;
  hdr[0] = ncow;
  hdr[1] = planned ? grid : 0;
  hdr[2] = ncut;
  hdr[3] = static_cast<int32_t>(lo.plan + plan_words);

  const int32_t* host_view = (reinterpret_cast<uintptr_t>(stage_host) | reinterpret_cast<uintptr_t>(stage_dev)) & 15u
                                 ? nullptr
                                 : device_view(stage_host, false);
  return run_device(fn, stage_host, host_view, stage_dev, n, table_stride, true, k_cache, v_cache, k_new, v_new, q,
                    out, out_dtype, kv_dtype, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                    partition_size, workspace, workspace_bytes, kernel, stream, 7, pass_begin, pass_end, d_times);
}

pa_status pa_step_layer(const int32_t* stage_host, int32_t* stage_dev, int32_t n, int32_t table_stride,
                        void* k_cache, void* v_cache, const void* k_new, const void* v_new, const void* q, void* out,
                        pa_dtype out_dtype, pa_dtype kv_dtype, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                        void* workspace, size_t workspace_bytes, pa_kernel kernel, void* stream, int32_t phases,
                        void* pass_begin, void* pass_end, int32_t* wave_times) {
  const char* fn = "pa_step_layer";
  if (!stage_host || !stage_dev || n <= 0 || table_stride <= 0 || phases < 1 || phases > 7)
    return pa::fail(PA_ERR_INVALID, "%s: bad arguments", fn);
  const Layout lo = layout(n, table_stride);
  const int32_t* hdr = stage_host + lo.header;
  const int32_t grid = pa::stream_grid_selected(kernel, kv_dtype, n, num_q_heads, num_kv_heads, head_dim);
  if (hdr[0] < 0 || hdr[0] > n || hdr[2] < 0 || hdr[2] > int64_t(n) * num_kv_heads ||
      size_t(hdr[3]) < lo.plan || (hdr[1] != 0 && hdr[1] != grid))
    return pa::fail(PA_ERR_INVALID, "%s: the record does not match this shape and kernel", fn);
  int32_t max_ctx = 0;
  for (int32_t i = 0; i < n; ++i) max_ctx = std::max(max_ctx, stage_host[3 * n + i]);
  if (pa_status st = pa::decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, stage_dev, table_stride,
                                     stage_dev, max_ctx, n, num_q_heads, num_kv_heads, head_dim, block_size,
                                     num_blocks, scale, partition_size, workspace, workspace_bytes, stream, kernel, 0,
                                     nullptr))
    return st;
  int32_t* d_times = nullptr;
  if (wave_times && !(d_times = device_view(wave_times, true)))
    return pa::fail(PA_ERR_INVALID, "%s: wave_times is neither pinned host nor device memory", fn);
  return run_device(fn, stage_host, nullptr, stage_dev, n, table_stride, false, k_cache, v_cache, k_new, v_new, q,
                    out, out_dtype, kv_dtype, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                    partition_size, workspace, workspace_bytes, kernel, stream, phases, pass_begin, pass_end,
                    d_times);
}

}  // extern "C"
