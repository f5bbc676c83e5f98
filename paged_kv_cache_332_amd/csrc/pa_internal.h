// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pa.h"

namespace pa {

// Records a printf-style message for pa_last_error() and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...);

// Optional inputs of the stream kernel (device pointers, each may be null):
// a host plan of its split and the wave stamp output.
struct StreamExtras {
  const int32_t* pre;          // [B + 1] tiles (16 tokens) of the sequences before each one
  const int32_t* wave_start;   // [grid * 4 + 1] first tile of each wave
  const int32_t* cut_entry;    // [num_cut][8] item code, wave count, offset, first four waves
  const int32_t* cut_workers;  // the waves of each cut item, in order
  int32_t num_cut;
  int32_t* wave_time;          // [grid * 4][2] wave start and end stamps, 10 ns units (written)
  const int32_t* shared;       // [B] leading blocks of each sequence that other sequences also hold
};

pa_status decode_impl(void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
                      pa_dtype kv_dtype, const int32_t* block_tables, int32_t table_stride,
                      const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                      int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream,
                      pa_kernel kernel, int phases, const StreamExtras* extras);

int32_t stream_grid(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);
// The stream kernel's grid when decode_impl would run it for `kernel`, else 0.
int32_t stream_grid_selected(pa_kernel kernel, pa_dtype kv_dtype, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim);

}  // namespace pa
