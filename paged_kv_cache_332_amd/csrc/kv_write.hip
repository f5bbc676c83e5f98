// KV append through a slot mapping and whole-block copies for copy-on-write.
//
// A request fills the block it holds and asks for another only when it is
// full ("Paged Attention: Virtual Memory for the KV Cache", §The fix borrowed
// from operating systems); a sharer that diverges gets its own copy of the
// block it is about to write (§Sharing comes almost for free).  Both are
// plain data movement, bound by HBM: the kernels read each source byte once
// and write each destination byte once.
#include <algorithm>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

// One workgroup per token.  K: the token's row of each head is D/X 16-byte
// chunks that land at stride BS*16 bytes (K tile [D/X][BS][X]).  V: each
// element lands at stride BS elements (V tile [D][BS]).  Source reads are
// fully coalesced; destination writes are the scatter the layout implies.
template <typename Bits>
__global__ __launch_bounds__(256) void write_kv_kernel(u32x4* __restrict__ kc,
                                                       Bits* __restrict__ vc,
                                                       const u32x4* __restrict__ kn,
                                                       const Bits* __restrict__ vn,
                                                       const int32_t* __restrict__ slots,
                                                       int32_t hkv, int32_t d, int32_t bs) {
  const int64_t t = blockIdx.x;
  const int32_t s = slots[t];
  if (s < 0) return;
  const int64_t blk = s / bs;
  const int32_t off = s % bs;
  const int32_t x = 16 / static_cast<int32_t>(sizeof(Bits));
  const int32_t cpr = d / x;                      // 16-byte chunks per head row
  const int32_t nk = hkv * cpr;
  for (int32_t i = threadIdx.x; i < nk; i += blockDim.x) {
    const int32_t h = i / cpr, c = i % cpr;
    kc[((blk * hkv + h) * cpr + c) * bs + off] = kn[t * nk + i];
  }
  const int32_t nv = hkv * d;
  for (int32_t i = threadIdx.x; i < nv; i += blockDim.x) {
    const int32_t h = i / d, e = i % d;
    vc[((blk * hkv + h) * d + e) * bs + off] = vn[t * nv + i];
  }
}

// grid (num_pairs, 2 * hkv): one workgroup copies one (K or V, head) tile of
// a block, BS*D elements, in 16-byte units.
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ kc,
                                                          u32x4* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t hkv, int32_t tile_chunks) {
  const int32_t p = blockIdx.x;
  const int32_t kv = blockIdx.y / hkv, h = blockIdx.y % hkv;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  u32x4* base = kv ? vc : kc;
  const u32x4* from = base + (src * hkv + h) * tile_chunks;
  u32x4* to = base + (dst * hkv + h) * tile_chunks;
  for (int32_t i = threadIdx.x; i < tile_chunks; i += blockDim.x) to[i] = from[i];
}

// One decode step's record and KV write in one launch, on the compute queue
// (no copy engine, so the kernels that follow wait for no cross-engine
// signal).  Workgroups [0, n) write token blockIdx.x like write_kv_kernel,
// taking its slot from the record in pinned host memory; the other
// workgroups copy the record (`words` int32) from host to device memory in
// 16-byte units.
template <typename Bits>
__global__ __launch_bounds__(256) void step_stage_kernel(const int32_t* __restrict__ rec_host,
                                                         int32_t* __restrict__ rec_dev, int64_t words, int32_t n,
                                                         u32x4* __restrict__ kc, Bits* __restrict__ vc,
                                                         const u32x4* __restrict__ kn, const Bits* __restrict__ vn,
                                                         int32_t hkv, int32_t d, int32_t bs, StageSlots sl) {
  if (blockIdx.x >= n) {
    const int64_t units = words / 4;                  // words is a multiple of 4
    const u32x4* src = reinterpret_cast<const u32x4*>(rec_host);
    u32x4* dst = reinterpret_cast<u32x4*>(rec_dev);
    for (int64_t i = int64_t(blockIdx.x - n) * blockDim.x + threadIdx.x; i < units;
         i += int64_t(gridDim.x - n) * blockDim.x)
      dst[i] = src[i];
    return;
  }
  const int64_t t = blockIdx.x;
  // the slot travels in the launch arguments when it fits (no host-memory
  // round trip before the writes), else it is read from the record
  const int32_t s = n <= kStageArgSlots ? sl.slot[t] : rec_host[t];
  if (s < 0) return;
  const int64_t blk = s / bs;
  const int32_t off = s % bs;
  const int32_t x = 16 / static_cast<int32_t>(sizeof(Bits));
  const int32_t cpr = d / x;
  const int32_t nk = hkv * cpr;
  for (int32_t i = threadIdx.x; i < nk; i += blockDim.x) {
    const int32_t h = i / cpr, c = i % cpr;
    kc[((blk * hkv + h) * cpr + c) * bs + off] = kn[t * nk + i];
  }
  const int32_t nv = hkv * d;
  for (int32_t i = threadIdx.x; i < nv; i += blockDim.x) {
    const int32_t h = i / d, e = i % d;
    vc[((blk * hkv + h) * d + e) * bs + off] = vn[t * nv + i];
  }
}

hipError_t launch_step_stage(const int32_t* rec_host, int32_t* rec_dev, int64_t words, int32_t n, void* k_cache,
                             void* v_cache, const void* k_new, const void* v_new, int32_t hkv, int32_t d,
                             int32_t bs, int32_t elem_bytes, const int32_t* slots_host, hipStream_t stream) {
  const int64_t units = words / 4;
  const int32_t copiers = static_cast<int32_t>(std::min<int64_t>(64, std::max<int64_t>(1, (units + 255) / 256)));
  dim3 grid(n + copiers), block(256);
  StageSlots sl;
  if (n <= kStageArgSlots) std::copy(slots_host, slots_host + n, sl.slot);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(step_stage_kernel<uint16_t>, grid, block, 0, stream, rec_host, rec_dev, words, n,
                       static_cast<u32x4*>(k_cache), static_cast<uint16_t*>(v_cache),
                       static_cast<const u32x4*>(k_new), static_cast<const uint16_t*>(v_new), hkv, d, bs, sl);
  } else {
    hipLaunchKernelGGL(step_stage_kernel<uint32_t>, grid, block, 0, stream, rec_host, rec_dev, words, n,
                       static_cast<u32x4*>(k_cache), static_cast<uint32_t*>(v_cache),
                       static_cast<const u32x4*>(k_new), static_cast<const uint32_t*>(v_new), hkv, d, bs, sl);
  }
  return hipGetLastError();
}

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t num_tokens, int32_t hkv, int32_t d,
                           int32_t bs, int32_t elem_bytes, hipStream_t stream) {
  dim3 grid(num_tokens), block(256);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(write_kv_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<uint16_t*>(v_cache),
                       static_cast<const u32x4*>(k_new), static_cast<const uint16_t*>(v_new), slots,
                       hkv, d, bs);
  } else {
    hipLaunchKernelGGL(write_kv_kernel<uint32_t>, grid, block, 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<uint32_t*>(v_cache),
                       static_cast<const u32x4*>(k_new), static_cast<const uint32_t*>(v_new), slots,
                       hkv, d, bs);
  }
  return hipGetLastError();
}

// Whole blocks (all kv heads, K and V) between the pools and host memory the
// device can address: block blocks[i] <-> host slot i ([n][units] 16-byte
// units per pool).  Grid (n, 2, chunks): y selects K or V.
__global__ __launch_bounds__(256) void swap_blocks_kernel(u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                          u32x4* __restrict__ hk, u32x4* __restrict__ hv,
                                                          const int32_t* __restrict__ blocks, int64_t units,
                                                          int32_t num_blocks, int32_t to_host) {
  const int64_t i = blockIdx.x;
  const int64_t b = blocks[i];
  if (b < 0 || b >= num_blocks) return;  // an id outside the pool moves nothing
  u32x4* dev = (blockIdx.y ? vc : kc) + b * units;
  u32x4* host = (blockIdx.y ? hv : hk) + i * units;
  for (int64_t u = int64_t(blockIdx.z) * blockDim.x + threadIdx.x; u < units; u += int64_t(gridDim.z) * blockDim.x) {
    if (to_host) host[u] = dev[u];
    else dev[u] = host[u];
  }
}

hipError_t launch_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v, const int32_t* blocks,
                              int32_t n, int64_t block_bytes, int32_t num_blocks, int32_t to_host,
                              hipStream_t stream) {
  const int64_t units = block_bytes / 16;
  const int32_t chunks = static_cast<int32_t>(std::min<int64_t>(16, (units + 255) / 256));
  dim3 grid(n, 2, chunks), block(256);
  hipLaunchKernelGGL(swap_blocks_kernel, grid, block, 0, stream, static_cast<u32x4*>(k_cache),
                     static_cast<u32x4*>(v_cache), static_cast<u32x4*>(host_k), static_cast<u32x4*>(host_v), blocks,
                     units, num_blocks, to_host);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                              int32_t hkv, int32_t d, int32_t bs, int32_t elem_bytes,
                              hipStream_t stream) {
  const int32_t tile_chunks = d * bs * elem_bytes / 16;
  dim3 grid(num_pairs, 2 * hkv), block(256);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, block, 0, stream, static_cast<u32x4*>(k_cache),
                     static_cast<u32x4*>(v_cache), pairs, hkv, tile_chunks);
  return hipGetLastError();
}

}  // namespace pa
