// Launchers of the gfx950 kernels (host-callable, defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace pa {

// Lets `kern` take `lds` bytes of dynamic LDS (above the default limit) on the
// current device; `done` (one per kernel instantiation) records the devices
// already set, so the attribute call runs once per device and thread-safely.
template <class K>
inline hipError_t allow_dynamic_lds(K kern, size_t lds, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Arguments of the decode partition pass and the merge pass.
struct DecodeArgs {
  void* out;                     // [B][Hq][D], fp32 or the kv dtype
  const void* q;                 // [B][Hq][D], kv dtype
  const void* k;                 // K pool
  const void* v;                 // V pool
  const int32_t* tables;         // [B][table_stride]
  const int32_t* ctx;            // [B]
  float* ws_m;                   // [B][Hq][pmax]  running max (log2 domain)
  float* ws_l;                   // [B][Hq][pmax]  sum of exp2(s - m)
  float* ws_acc;                 // [B][Hq][pmax][D] unnormalised output
  int32_t table_stride;
  int32_t max_ctx;               // host bound; device lengths are clamped to [0, max_ctx]
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t pmax;                  // partitions of the longest context
  int32_t part;                  // tokens per partition
  float scale_log2;              // scale * log2(e)
  int32_t out_f32;               // 1: fp32 output, 0: kv dtype output
};

// Arguments of the stream kernel: the decode arguments plus its workspace.
struct StreamArgs {
  DecodeArgs d;
  float* rec_ml;                 // [workers][2][gmax][2]  (max, sum) of partial states
  float* rec_acc;                // [workers][2][gmax][D]  unnormalised partial outputs
  // optional host plan (all null: the kernels derive an equal split themselves)
  const int32_t* pre_in;         // [B + 1] tiles of the sequences before each one
  const int32_t* wave_start;     // [grid * 4 + 1] first tile of each wave, non-decreasing, last = all tiles
  const int32_t* cut_entry;      // [num_cut][8] {2 * (seq * Hkv + kvh) + (1 if its first wave starts before
                                 // it), its wave count, offset in cut_workers, first four waves}
  const int32_t* cut_workers;    // waves with tiles of each cut item, in order
  int32_t num_cut;
  int32_t* wave_time;            // [grid * 4][2] start and end of each wave (low 32 bits of the
                                 // 100 MHz real-time counter), or null
  const int32_t* shared;         // [B] leading blocks of each sequence that other sequences also
                                 // hold (read again in the same pass), or null: none
};

// Stream kernel limits: tiles whose block ids a wave stages per pass, the
// largest batch, and its static LDS (block ids, lengths, prefix sums).
constexpr int kStreamTcap = 224;
constexpr int kStreamMaxGrid = 1024;      // workgroups of one stream launch
constexpr int kStreamMaxSeqs = 1024;
// (16 KiB bounds the arrays with the compiler's alignment padding)
constexpr size_t kStreamStaticLds = 16 * 1024;
static_assert(4 * kStreamTcap * 8 + (2 * kStreamMaxSeqs + 1) * 4 + 64 <= kStreamStaticLds, "static LDS");
constexpr size_t kStreamLdsPerCu = 160 * 1024;

// Dynamic LDS bytes (the tile rings) of one stream workgroup.
size_t stream_lds_bytes(int d, int gmax, int nslot);
// phases: bit 0 the stream pass, bit 1 the merge of cut items
hipError_t launch_decode_stream(const StreamArgs& sa, int32_t dtype, int32_t d, int32_t bs, int32_t gmax,
                                int32_t nslot, size_t lds, int32_t grid, int32_t phases, hipStream_t stream);

// Arguments of the paged prefill kernel.
struct PrefillArgs {
  void* out;                     // [T][Hq][D], fp32 or the kv dtype (T = query rows of all chunks)
  const void* q;                 // [T][Hq][D], kv dtype
  const void* k;                 // K pool
  const void* v;                 // V pool
  const int32_t* tables;         // [B][table_stride]
  const int32_t* query_start;    // [B + 1] first query row of each sequence's chunk
  const int32_t* ctx;            // [B] context length including the chunk
  int32_t table_stride;
  int32_t max_ctx;               // host bound; device lengths are clamped to it
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  float scale_log2;              // scale * log2(e)
  int32_t out_f32;
};
// Column blocks per prefill wave (16 / group tokens each): more blocks
// share each streamed tile and K operand among more columns, fewer keep
// short chunks spread over enough workgroups.  3 when that leaves at least
// 1024 workgroups and rounding the longest chunk up to whole query blocks of
// 12 (16 / group) tokens pads at most a fifth of the rounded rows, 2 when
// that leaves at least 512 and blocks of 8 (16 / group) tokens pad at most a
// fifth, else 1 (a chunk shorter than one block takes neither).
inline int32_t prefill_column_blocks(int32_t group, int32_t max_query_len, int32_t num_seqs, int32_t num_kv_heads) {
  auto wgs = [&](int64_t cb) {
    const int64_t tpw = 4 * cb * (16 / group);
    return max_query_len < tpw ? int64_t(0) : int64_t(num_seqs) * num_kv_heads * ((max_query_len + tpw - 1) / tpw);
  };
  const int64_t tpw3 = 12 * (16 / group);
  const int64_t rows3 = (int64_t(max_query_len) + tpw3 - 1) / tpw3 * tpw3;
  if (wgs(3) >= 1024 && 5 * (rows3 - max_query_len) <= rows3) return 3;
  const int64_t tpw2 = 8 * (16 / group);
  const int64_t rows2 = (int64_t(max_query_len) + tpw2 - 1) / tpw2 * tpw2;
  return wgs(2) >= 512 && 5 * (rows2 - max_query_len) <= rows2 ? 2 : 1;
}
hipError_t launch_prefill(const PrefillArgs& a, int32_t dtype, int32_t d, int32_t bs, int32_t group,
                          int32_t max_query_len, hipStream_t stream);

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t num_tokens, int32_t hkv, int32_t d,
                           int32_t bs, int32_t elem_bytes, hipStream_t stream);

// Step record copy (pinned host -> device, `words` a multiple of 4) fused with
// the KV write of its n tokens (slots = the record's first n words; up to
// kStageArgSlots of them, read on the host through slots_host, travel in the
// launch arguments).
constexpr int kStageArgSlots = 512;
struct StageSlots {
  int32_t slot[kStageArgSlots];
};
hipError_t launch_step_stage(const int32_t* rec_host, int32_t* rec_dev, int64_t words, int32_t n, void* k_cache,
                             void* v_cache, const void* k_new, const void* v_new, int32_t hkv, int32_t d,
                             int32_t bs, int32_t elem_bytes, const int32_t* slots_host, hipStream_t stream);

// block_bytes = bytes of one block of one pool (all kv heads), a multiple of
// 16; ids outside [0, num_blocks) are skipped
hipError_t launch_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v, const int32_t* blocks,
                              int32_t n, int64_t block_bytes, int32_t num_blocks, int32_t to_host,
                              hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                              int32_t hkv, int32_t d, int32_t bs, int32_t elem_bytes,
                              hipStream_t stream);

// dtype: 0 f32, 1 f16, 2 bf16 (pa_dtype values).  Return hipErrorInvalidValue
// for a shape they were not instantiated for.
hipError_t launch_decode_valu(const DecodeArgs& a, int32_t dtype, int32_t d, int32_t bs,
                              int32_t group, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, int32_t dtype, int32_t d, int32_t bs,
                              int32_t group, hipStream_t stream);
hipError_t launch_merge(const DecodeArgs& a, int32_t dtype, int32_t d, hipStream_t stream);

}  // namespace pa
