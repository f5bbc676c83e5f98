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
#include <cstdint>

#include "pa_internal.h"
#include "pa_kernels.h"

namespace {

// Device-visible address of pinned host memory (the same address on a
// unified address space), or nullptr when the runtime reports none.  The
// last few lookups are cached: callers rotate a handful of step records.
const int32_t* device_view(const int32_t* host) {
  struct Entry {
    const void* host;
    const void* dev;
  };
  static thread_local Entry cache[8] = {};
  static thread_local int next = 0;
  for (const Entry& e : cache)
    if (e.host == host) return static_cast<const int32_t*>(e.dev);
  hipPointerAttribute_t attr{};
  const void* dev = nullptr;
  if (hipPointerGetAttributes(&attr, host) == hipSuccess && attr.type == hipMemoryTypeHost && attr.devicePointer)
    dev = attr.devicePointer;
  (void)hipGetLastError();  // a plain host pointer leaves an error behind
  cache[next] = Entry{host, dev};
  next = (next + 1) % 8;
  return static_cast<const int32_t*>(dev);
}

}  // namespace

extern "C" {

pa_status pa_step(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* stage_host, int32_t* stage_dev,
                  int32_t table_stride, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  const void* q, void* out, pa_dtype out_dtype, pa_dtype kv_dtype, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                  int32_t partition_size, void* workspace, size_t workspace_bytes, pa_kernel kernel,
                  void* stream, void* pass_begin, void* pass_end, int32_t* max_ctx_out) {
  const char* fn = "pa_step";
  if (!bm || !seqs || !stage_host || !stage_dev || n <= 0 || table_stride <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_INVALID, "%s: bad arguments", fn);
  // every sequence must still fit the table stride after its new token, so
  // that the export below cannot fail once the manager has changed
  for (int32_t i = 0; i < n; ++i) {
    const int32_t len = pa_bm_seq_len(bm, seqs[i]);
    if (len < 0) return pa::fail(PA_ERR_INVALID, "%s: unknown sequence %lld", fn, static_cast<long long>(seqs[i]));
    if (static_cast<int64_t>(len) + 1 > static_cast<int64_t>(table_stride) * block_size)
      return pa::fail(PA_ERR_INVALID, "%s: sequence %lld outgrows the table stride %d", fn,
                      static_cast<long long>(seqs[i]), table_stride);
  }
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

  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t words = (4 * static_cast<size_t>(n) + static_cast<size_t>(n) * table_stride + 3) / 4 * 4;
  const int32_t* host_view = (reinterpret_cast<uintptr_t>(stage_host) | reinterpret_cast<uintptr_t>(stage_dev)) & 15u
                                 ? nullptr
                                 : device_view(stage_host);
  if (host_view) {
    // the kernels read the record where the host wrote it: copy-on-write
    // copies, then one launch that copies the record to the device and
    // writes the new tokens' keys and values
    if (ncow) {
      if (pa_status st = pa_copy_blocks(k_cache, v_cache, host_view + n, ncow, num_kv_heads, head_dim, block_size,
                                        num_blocks, kv_dtype, stream))
        return st;
    }
    if (pa_status st = pa_write_kv(k_cache, v_cache, k_new, v_new, stage_dev, 0, num_kv_heads, head_dim, block_size,
                                   num_blocks, kv_dtype, stream))
      return st;  // validates the cache arguments; writes nothing
    if (!k_new || !v_new || (reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15u)
      return pa::fail(PA_ERR_INVALID, "%s: k_new and v_new must be 16-byte aligned device memory", fn);
    if (hipError_t e = pa::launch_step_stage(host_view, stage_dev, static_cast<int64_t>(words), n, k_cache, v_cache,
                                             k_new, v_new, num_kv_heads, head_dim, block_size,
                                             kv_dtype == PA_F32 ? 4 : 2, s))
      return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  } else {
    if (hipError_t e = hipMemcpyAsync(stage_dev, stage_host, words * sizeof(int32_t), hipMemcpyHostToDevice, s))
      return pa::fail(PA_ERR_HIP, "%s: copy of the step record: %s", fn, hipGetErrorString(e));
    if (ncow) {
      if (pa_status st = pa_copy_blocks(k_cache, v_cache, stage_dev + n, ncow, num_kv_heads, head_dim, block_size,
                                        num_blocks, kv_dtype, stream))
        return st;
    }
    if (pa_status st = pa_write_kv(k_cache, v_cache, k_new, v_new, stage_dev, n, num_kv_heads, head_dim,
                                   block_size, num_blocks, kv_dtype, stream))
      return st;
  }
  if (pass_begin) {
    if (hipError_t e = hipEventRecord(static_cast<hipEvent_t>(pass_begin), s))
      return pa::fail(PA_ERR_HIP, "%s: event: %s", fn, hipGetErrorString(e));
  }
  const int32_t* d_ctx = stage_dev + 3 * n;
  const int32_t* d_tables = stage_dev + 4 * n;
  if (pa_status st = pa_decode_phase(out, out_dtype, q, k_cache, v_cache, kv_dtype, d_tables, table_stride, d_ctx,
                                     max_ctx, n, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                                     partition_size, workspace, workspace_bytes, stream, kernel, PA_PHASE_PASS))
    return st;
  if (pass_end) {
    if (hipError_t e = hipEventRecord(static_cast<hipEvent_t>(pass_end), s))
      return pa::fail(PA_ERR_HIP, "%s: event: %s", fn, hipGetErrorString(e));
  }
  return pa_decode_phase(out, out_dtype, q, k_cache, v_cache, kv_dtype, d_tables, table_stride, d_ctx, max_ctx, n,
                         num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                         workspace, workspace_bytes, stream, kernel, PA_PHASE_MERGE);
}

}  // extern "C"
