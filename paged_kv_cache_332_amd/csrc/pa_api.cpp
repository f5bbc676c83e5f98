// C ABI of libpa.so: argument validation, kernel selection and launches.
// The operations and their citations are documented in include/pa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "pa_internal.h"
#include "pa_kernels.h"
#include "prefill_split.h"

namespace pa {

namespace {
thread_local std::string g_error;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }
bool valid_dtype(pa_dtype d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The pointer itself if the device can address it: device memory, or pinned
// host memory mapped at the same address on the device (one unified address
// space); nullptr otherwise.
void* device_address(const void* p) {
  hipPointerAttribute_t attr{};
  void* dev = nullptr;
  if (hipPointerGetAttributes(&attr, p) == hipSuccess) {
    if (attr.type == hipMemoryTypeHost && attr.devicePointer && attr.devicePointer == attr.hostPointer) {
      dev = const_cast<void*>(p);
    } else if (attr.type == hipMemoryTypeDevice) {
      dev = const_cast<void*>(p);
    }
  }
  (void)hipGetLastError();  // a plain host pointer leaves an error behind
  return dev;
}

pa_status check_cache_shape(const char* fn, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, pa_dtype dtype) {
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID, "%s: unknown dtype %d", fn, int(dtype));
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID, "%s: sizes must be positive (heads %d, dim %d, block %d, blocks %d)", fn,
                num_kv_heads, head_dim, block_size, num_blocks);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d not in {8, 16, 32}", fn, block_size);
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PA_ERR_INVALID, "%s: num_blocks * block_size must stay below 2^31", fn);
  return PA_OK;
}

pa_status hip_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
}

int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

constexpr int32_t kMinAutoPartition = 256;

}  // namespace

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

}  // namespace pa

extern "C" {

const char* pa_last_error(void) { return pa::g_error.c_str(); }

const char* pa_version(void) { return "pa 0.1 gfx950"; }

pa_status pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                      void* stream) {
  if (pa_status st = pa::check_cache_shape("pa_write_kv", num_kv_heads, head_dim, block_size, num_blocks, dtype))
    return st;
  if (num_tokens < 0) return pa::fail(PA_ERR_INVALID, "pa_write_kv: num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return pa::fail(PA_ERR_INVALID, "pa_write_kv: null pointer");
  if (!pa::aligned16(k_cache) || !pa::aligned16(k_new) || !pa::aligned16(v_cache) || !pa::aligned16(v_new))
    return pa::fail(PA_ERR_INVALID, "pa_write_kv: caches and inputs must be 16-byte aligned");
  return pa::hip_status("pa_write_kv",
                        pa::launch_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens,
                                            num_kv_heads, head_dim, block_size, pa::elem_bytes(dtype),
                                            static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, pa_dtype dtype, void* stream) {
  if (pa_status st = pa::check_cache_shape("pa_copy_blocks", num_kv_heads, head_dim, block_size, num_blocks, dtype))
    return st;
  if (num_pairs < 0) return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: null pointer");
  if (!pa::aligned16(k_cache) || !pa::aligned16(v_cache))
    return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: caches must be 16-byte aligned");
  if (2 * num_kv_heads > 65535) return pa::fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: too many kv heads");
  return pa::hip_status("pa_copy_blocks",
                        pa::launch_copy_blocks(k_cache, v_cache, pairs, num_pairs, num_kv_heads, head_dim,
                                               block_size, pa::elem_bytes(dtype),
                                               static_cast<hipStream_t>(stream)));
}

pa_status pa_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v, const int32_t* blocks,
                         int32_t num_blocks_moved, int32_t to_host, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
  const char* fn = "pa_swap_blocks";
  if (pa_status st = pa::check_cache_shape(fn, num_kv_heads, head_dim, block_size, num_blocks, dtype)) return st;
  if (num_blocks_moved < 0 || (to_host != 0 && to_host != 1))
    return pa::fail(PA_ERR_INVALID, "%s: bad arguments", fn);
  if (num_blocks_moved == 0) return PA_OK;
  if (!k_cache || !v_cache || !host_k || !host_v || !blocks) return pa::fail(PA_ERR_INVALID, "%s: null pointer", fn);
  if (!pa::aligned16(k_cache) || !pa::aligned16(v_cache) || !pa::aligned16(host_k) || !pa::aligned16(host_v))
    return pa::fail(PA_ERR_INVALID, "%s: caches and host buffers must be 16-byte aligned", fn);
  // the host buffers and the list must be addressable by the device: pinned
  // host memory (its device address is used) or device memory
  void* hk = pa::device_address(host_k);
  void* hv = pa::device_address(host_v);
  const int32_t* bl = static_cast<const int32_t*>(pa::device_address(blocks));
  if (!hk || !hv || !bl)
    return pa::fail(PA_ERR_INVALID, "%s: host buffers and the block list must be pinned host or device memory", fn);
  const int64_t block_bytes = int64_t(num_kv_heads) * head_dim * block_size * pa::elem_bytes(dtype);
  return pa::hip_status(fn, pa::launch_swap_blocks(k_cache, v_cache, hk, hv, bl, num_blocks_moved, block_bytes,
                                                   num_blocks, to_host, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                    int32_t block_size) {
  (void)num_seqs;
  (void)max_context_len;
  (void)block_size;
  return 512;
}

}  // extern "C"

namespace pa {
namespace {

// Stream-kernel plan for a shape: slots per wave, LDS bytes, grid size.
struct StreamPlan {
  int gmax = 0, nslot = 0, grid = 0;
  size_t lds = 0;
  size_t ml_bytes = 0, acc_bytes = 0;
  bool ok = false;
};


// Compute units of the current device, looked up once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    if (const int c = cache[dev].load(std::memory_order_relaxed)) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  if (dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

StreamPlan stream_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t head_dim) {
  StreamPlan p;
  p.gmax = group <= 4 ? 4 : group <= 8 ? 8 : 16;
  if (num_seqs > kStreamMaxSeqs) return p;
  for (int ns = 4; ns >= 2; --ns) {
    const size_t lds = stream_lds_bytes(head_dim, p.gmax, ns);
    if (lds + kStreamStaticLds <= kStreamLdsPerCu) {
      p.nslot = ns;
      p.lds = lds;
      break;
    }
  }
  if (!p.nslot) return p;
  const int per_cu = static_cast<int>(kStreamLdsPerCu / (p.lds + kStreamStaticLds));
  p.grid = std::min(kStreamMaxGrid, device_cus() * std::max(1, per_cu));
  const size_t workers = size_t(p.grid) * 4;
  p.ml_bytes = round_up(workers * 2 * p.gmax * 2 * sizeof(float));
  p.acc_bytes = round_up(workers * 2 * p.gmax * size_t(head_dim) * sizeof(float));
  p.ok = true;
  return p;
}

size_t partition_ws_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t pmax) {
  if (pmax <= 1) return 0;
  const size_t rows = size_t(num_seqs) * num_q_heads * pmax;
  return 2 * round_up(rows * sizeof(float)) + round_up(rows * head_dim * sizeof(float));
}

}  // namespace
}  // namespace pa

extern "C" {

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
      max_context_len < 0 || partition_size < 0)
    return 0;
  const int32_t part = partition_size ? partition_size : pa::kMinAutoPartition;
  const int32_t pmax = std::max(1, pa::ceil_div(max_context_len, part));
  size_t need = pa::partition_ws_bytes(num_seqs, num_q_heads, head_dim, pmax);
  const pa::StreamPlan sp = pa::stream_plan(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim);
  if (sp.ok) need = std::max(need, sp.ml_bytes + sp.acc_bytes);
  return need;
}

}  // extern "C"

namespace pa {

// Validates, picks the kernel and launches the phases asked for (bit 0: the
// pass over the K/V tiles, bit 1: the merge of split items; 0 validates
// only).  `extras` (may be null) passes the stream kernel's host plan and
// the wave stamp output.
pa_status decode_impl(void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
                      pa_dtype kv_dtype, const int32_t* block_tables, int32_t table_stride,
                      const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream,
                      pa_kernel kernel, int phases, const StreamExtras* extras) {
  const char* fn = "pa_decode";
  if (phases < 0 || phases > 3) return pa::fail(PA_ERR_INVALID, "%s: phases %d not in 1..3", fn, phases);
  if (pa_status st = pa::check_cache_shape(fn, num_kv_heads, head_dim, block_size, num_blocks, kv_dtype))
    return st;
  if (out_dtype != PA_F32 && out_dtype != kv_dtype)
    return pa::fail(PA_ERR_INVALID, "%s: out_dtype must be F32 or the kv dtype", fn);
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || table_stride < 0)
    return pa::fail(PA_ERR_INVALID, "%s: bad sizes (seqs %d, q heads %d, max ctx %d, stride %d)", fn, num_seqs,
                    num_q_heads, max_context_len, table_stride);
  if (num_q_heads % num_kv_heads)
    return pa::fail(PA_ERR_INVALID, "%s: %d query heads not a multiple of %d kv heads", fn, num_q_heads,
                    num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: group size %d not in {1,2,4,8,16}", fn, group);
  if (pa::ceil_div(max_context_len, block_size) > table_stride)
    return pa::fail(PA_ERR_INVALID, "%s: table_stride %d < blocks of max_context_len %d", fn, table_stride,
                    max_context_len);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return pa::fail(PA_ERR_INVALID, "%s: null pointer", fn);
  if (!pa::aligned16(q) || !pa::aligned16(k_cache) || !pa::aligned16(v_cache))
    return pa::fail(PA_ERR_INVALID, "%s: q and caches must be 16-byte aligned", fn);
  if (kernel != PA_KERNEL_AUTO && kernel != PA_KERNEL_VALU && kernel != PA_KERNEL_MFMA &&
      kernel != PA_KERNEL_STREAM)
    return pa::fail(PA_ERR_INVALID, "%s: unknown kernel %d", fn, int(kernel));
  if ((kernel == PA_KERNEL_MFMA || kernel == PA_KERNEL_STREAM) && kv_dtype == PA_F32)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: the matrix-core kernels need a 16-bit cache", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kernel == PA_KERNEL_STREAM || (kernel == PA_KERNEL_AUTO && kv_dtype != PA_F32)) {
    const pa::StreamPlan sp = pa::stream_plan(num_seqs, num_kv_heads, group, head_dim);
    if (sp.ok) {
      const size_t need = sp.ml_bytes + sp.acc_bytes;
      if (!workspace || workspace_bytes < need)
        return pa::fail(PA_ERR_INVALID, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace_bytes);
      if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return pa::fail(PA_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
      // tile positions within a sequence's kv heads are 32-bit
      if (int64_t(num_kv_heads) * pa::ceil_div(max_context_len, 16) >= (int64_t(1) << 31))
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: context too long for the stream kernel", fn);
      if (phases == 0) return PA_OK;
      pa::StreamArgs sa{};
      sa.d.out = out;
      sa.d.q = q;
      sa.d.k = k_cache;
      sa.d.v = v_cache;
      sa.d.tables = block_tables;
      sa.d.ctx = context_lens;
      sa.d.table_stride = table_stride;
      sa.d.max_ctx = max_context_len;
      sa.d.num_seqs = num_seqs;
      sa.d.num_q_heads = num_q_heads;
      sa.d.num_kv_heads = num_kv_heads;
      sa.d.pmax = 1;
      sa.d.part = 0;
      sa.d.scale_log2 = scale * 1.4426950408889634f;
      sa.d.out_f32 = out_dtype == PA_F32;
      char* w = static_cast<char*>(workspace);
      sa.rec_ml = reinterpret_cast<float*>(w);
      sa.rec_acc = reinterpret_cast<float*>(w + sp.ml_bytes);
      if (extras) {
        sa.pre_in = extras->pre;
        sa.wave_start = extras->wave_start;
        sa.cut_entry = extras->cut_entry;
        sa.cut_workers = extras->cut_workers;
        sa.num_cut = extras->num_cut;
        sa.wave_time = extras->wave_time;
        sa.shared = extras->shared;
      }
      return pa::hip_status(fn, pa::launch_decode_stream(sa, kv_dtype, head_dim, block_size, sp.gmax, sp.nslot,
                                                          sp.lds, sp.grid, phases, s));
    }
    if (kernel == PA_KERNEL_STREAM)
      return pa::fail(PA_ERR_UNSUPPORTED, "%s: %d sequences do not fit the stream kernel's LDS", fn, num_seqs);
  }
  const int32_t part = partition_size ? partition_size
                                      : pa_decode_default_partition(num_seqs, num_kv_heads, max_context_len,
                                                                    block_size);
  if (part <= 0 || part % 64 || part % (4 * block_size))
    return pa::fail(PA_ERR_INVALID, "%s: partition_size %d must be a positive multiple of 64 and of 4*BS", fn,
                    part);
  const int32_t pmax = std::max(1, pa::ceil_div(max_context_len, part));
  if (static_cast<int64_t>(num_kv_heads) * pmax * num_seqs * (group > 4 && kernel == PA_KERNEL_VALU ? group / 4 : 1) >=
      (int64_t(1) << 31) - 8)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: too many work items", fn);
  size_t need = 0;
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.table_stride = table_stride;
  a.max_ctx = max_context_len;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.pmax = pmax;
  a.part = part;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_f32 = out_dtype == PA_F32;
  if (pmax > 1) {
    const size_t rows = size_t(num_seqs) * num_q_heads * pmax;
    const size_t ml = pa::round_up(rows * sizeof(float));
    need = 2 * ml + pa::round_up(rows * head_dim * sizeof(float));
    if (!workspace || workspace_bytes < need)
      return pa::fail(PA_ERR_INVALID, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
    char* w = static_cast<char*>(workspace);
    a.ws_m = reinterpret_cast<float*>(w);
    a.ws_l = reinterpret_cast<float*>(w + ml);
    a.ws_acc = reinterpret_cast<float*>(w + 2 * ml);
  }
  if (phases == 0) return PA_OK;
  const bool use_mfma = kernel == PA_KERNEL_MFMA || (kernel == PA_KERNEL_AUTO && kv_dtype != PA_F32);
  if (phases & 1) {
    hipError_t e = use_mfma ? pa::launch_decode_mfma(a, kv_dtype, head_dim, block_size, group, s)
                            : pa::launch_decode_valu(a, kv_dtype, head_dim, block_size, group, s);
    if (e != hipSuccess) return pa::hip_status(fn, e);
  }
  if ((phases & 2) && pmax > 1) {
    hipError_t e = pa::launch_merge(a, kv_dtype, head_dim, s);
    if (e != hipSuccess) return pa::hip_status(fn, e);
  }
  return PA_OK;
}

int32_t stream_grid(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return 0;
  const StreamPlan sp = stream_plan(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim);
  return sp.ok ? sp.grid : 0;
}

int32_t stream_grid_selected(pa_kernel kernel, pa_dtype kv_dtype, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim) {
  const bool stream = kernel == PA_KERNEL_STREAM || (kernel == PA_KERNEL_AUTO && kv_dtype != PA_F32);
  return stream ? stream_grid(num_seqs, num_q_heads, num_kv_heads, head_dim) : 0;
}

}  // namespace pa

extern "C" {

int32_t pa_decode_stream_grid(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  return pa::stream_grid(num_seqs, num_q_heads, num_kv_heads, head_dim);
}

pa_status pa_decode_variant(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                            const void* v_cache, pa_dtype kv_dtype, const int32_t* block_tables,
                            int32_t table_stride, const int32_t* context_lens, int32_t max_context_len,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, void* stream, pa_kernel kernel) {
  return pa::decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, table_stride, context_lens,
                         max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         scale, partition_size, workspace, workspace_bytes, stream, kernel, 3, nullptr);
}

pa_status pa_decode_phase(void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
                          pa_dtype kv_dtype, const int32_t* block_tables, int32_t table_stride,
                          const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, float scale, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, void* stream, pa_kernel kernel, int32_t phase) {
  if (phase < 1 || phase > 3) return pa::fail(PA_ERR_INVALID, "pa_decode: phase %d not in 1..3", int(phase));
  return pa::decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, table_stride, context_lens,
                         max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         scale, partition_size, workspace, workspace_bytes, stream, kernel, phase, nullptr);
}

pa_status pa_prefill(void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
                     pa_dtype kv_dtype, const int32_t* block_tables, int32_t table_stride,
                     const int32_t* query_start, const int32_t* context_lens, int32_t max_query_len,
                     int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const char* fn = "pa_prefill";
  if (pa_status st = pa::check_cache_shape(fn, num_kv_heads, head_dim, block_size, num_blocks, kv_dtype)) return st;
  if (kv_dtype == PA_F32) return pa::fail(PA_ERR_UNSUPPORTED, "%s: the prefill kernel needs a 16-bit cache", fn);
  if (out_dtype != PA_F32 && out_dtype != kv_dtype)
    return pa::fail(PA_ERR_INVALID, "%s: out_dtype must be F32 or the kv dtype", fn);
  if (num_seqs < 0 || num_q_heads <= 0 || max_query_len < 0 || max_context_len < 0 || table_stride < 0)
    return pa::fail(PA_ERR_INVALID, "%s: bad sizes", fn);
  if (num_q_heads % num_kv_heads)
    return pa::fail(PA_ERR_INVALID, "%s: %d query heads not a multiple of %d kv heads", fn, num_q_heads,
                    num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: group size %d not in {1,2,4,8,16}", fn, group);
  if (max_query_len > max_context_len)
    return pa::fail(PA_ERR_INVALID, "%s: max_query_len %d exceeds max_context_len %d", fn, max_query_len,
                    max_context_len);
  if (pa::ceil_div(max_context_len, block_size) > table_stride)
    return pa::fail(PA_ERR_INVALID, "%s: table_stride %d < blocks of max_context_len %d", fn, table_stride,
                    max_context_len);
  if (int64_t(num_seqs) * num_kv_heads > 65535)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: more than 65535 (sequence, kv head) pairs", fn);
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start || !context_lens)
    return pa::fail(PA_ERR_INVALID, "%s: null pointer", fn);
  if (!pa::aligned16(q) || !pa::aligned16(k_cache) || !pa::aligned16(v_cache) || !pa::aligned16(out))
    return pa::fail(PA_ERR_INVALID, "%s: q, out and caches must be 16-byte aligned", fn);
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.query_start = query_start;
  a.ctx = context_lens;
  a.table_stride = table_stride;
  a.max_ctx = max_context_len;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_f32 = out_dtype == PA_F32;
  pa::PrefillSplitArgs sa;
  if (workspace) {
    const pa::PrefillSplit sp = pa::prefill_split(group, max_query_len, max_context_len, num_seqs, num_q_heads,
                                                  num_kv_heads, head_dim);
    if (sp.split_tiles) {
      if (workspace_bytes < sp.bytes)
        return pa::fail(PA_ERR_INVALID, "%s: workspace of %zu bytes, the context split needs %zu", fn,
                        workspace_bytes, sp.bytes);
      if (!pa::aligned16(workspace)) return pa::fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
      sa.split_tiles = sp.split_tiles;
      sa.split_max = sp.split_max;
      sa.rows_per_seq = sp.rows_per_seq;
      sa.ws_ml = static_cast<float*>(workspace);
      sa.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + sp.ml_bytes);
    }
  }
  return pa::hip_status(fn, pa::launch_prefill_split(a, sa, kv_dtype, head_dim, block_size, group, max_query_len,
                                                     static_cast<hipStream_t>(stream)));
}

int32_t pa_prefill_column_blocks(int32_t num_q_heads, int32_t num_kv_heads, int32_t max_query_len, int32_t num_seqs) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || max_query_len < 0 || num_seqs < 0)
    return 0;
  const int32_t group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16) return 0;
  return pa::prefill_column_blocks(group, max_query_len, num_seqs, num_kv_heads);
}

size_t pa_prefill_workspace_bytes(int32_t max_query_len, int32_t max_context_len, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  if (max_query_len <= 0 || max_context_len <= 0 || num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || num_q_heads % num_kv_heads)
    return 0;
  const int32_t group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16) return 0;
  return pa::prefill_split(group, max_query_len, max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim)
      .bytes;
}

pa_status pa_decode(void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
                    pa_dtype kv_dtype, const int32_t* block_tables, int32_t table_stride,
                    const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, float scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return pa_decode_variant(out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, table_stride,
                           context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           block_size, num_blocks, scale, partition_size, workspace, workspace_bytes, stream,
                           PA_KERNEL_AUTO);
}

}  // extern "C"

// ---------------------------------------------------- allocation-free decode
namespace {

// The decode workspace of pa_decode_noalloc: a fixed array in device memory,
// one copy per device, held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device array: host code passes the
// device address hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = PA_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kScratchDevices = 64;

// Device address of the current device's scratch copy (null with *err set
// when the lookup fails).
void* scratch_on_current_device(hipError_t* err) {
  static std::once_flag once[kScratchDevices];
  static void* ptr[kScratchDevices];
  static hipError_t status[kScratchDevices];
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kScratchDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(once[dev], [dev] { status[dev] = hipGetSymbolAddress(&ptr[dev], HIP_SYMBOL(scratch)); });
  *err = status[dev];
  return status[dev] == hipSuccess ? ptr[dev] : nullptr;
}

// Workspace bytes the kernel pa_decode picks for these arguments uses (the
// stream kernel's per-wave records, or the partition kernels' partials when
// a sequence spans several partitions).
size_t selected_workspace_bytes(pa_dtype kv_dtype, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len, int32_t block_size, int32_t partition_size) {
  if (kv_dtype != PA_F32) {
    const pa::StreamPlan sp = pa::stream_plan(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim);
    if (sp.ok) return sp.ml_bytes + sp.acc_bytes;
  }
  const int32_t part = partition_size ? partition_size
                                      : pa_decode_default_partition(num_seqs, num_kv_heads, max_context_len,
                                                                    block_size);
  if (part <= 0) return 0;  // rejected by the validation that follows
  return pa::partition_ws_bytes(num_seqs, num_q_heads, head_dim, std::max(1, pa::ceil_div(max_context_len, part)));
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                                       const void* v_cache, pa_dtype kv_dtype, const int32_t* block_tables,
                                       int32_t table_stride, const int32_t* context_lens, int32_t max_context_len,
                                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                                       void* stream) {
  const char* fn = "pa_decode_noalloc";
  // the sizes the workspace depends on; anything else is left to pa_decode's
  // own validation below
  if (num_seqs > 0 && num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 && head_dim > 0 &&
      max_context_len >= 0 && block_size > 0 && partition_size >= 0) {
    const size_t need = selected_workspace_bytes(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_context_len, block_size, partition_size);
    if (need > kScratchBytes)
      return pa::fail(PA_ERR_INVALID,
                      "%s: this call needs %zu bytes of decode workspace, more than the %zu bytes of static "
                      "scratch (use pa_decode with a workspace)",
                      fn, need, kScratchBytes);
  }
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (!ws) return pa::fail(PA_ERR_HIP, "%s: address of the static scratch: %s", fn, hipGetErrorString(e));
  return pa::decode_impl(out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, table_stride, context_lens,
                         max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         scale, partition_size, ws, kScratchBytes, stream, PA_KERNEL_AUTO, 3, nullptr);
}
