// Context split of a paged prefill launch: its arguments, the host rule that
// chooses it and the launch that takes it (prefill.hip, pa_api.cpp).
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "pa_kernels.h"

namespace pa {

// Partial states of piece z of sequence s, query token t, head h sit at
// ((z B + s) rows_per_seq + t) Hq + h (split_tiles 0: no split).
struct PrefillSplitArgs {
  int32_t split_tiles = 0;       // tiles per piece (even)
  int32_t split_max = 1;         // pieces of the longest context
  int32_t rows_per_seq = 0;      // query tokens the grid covers per sequence
  float* ws_ml = nullptr;        // (reference maximum, sum) pairs
  float* ws_acc = nullptr;       // unnormalised outputs, D floats each
};

// A launch of fewer than kPrefillSplitBelow workgroups (two per compute
// unit: short chunks of few sequences, where one workgroup streams a whole
// context and most compute units idle) splits each sequence's prefix into
// pieces of split_tiles tiles, at least kPrefillMinSplitTiles (a piece's
// partial states, 520 bytes per column at D = 128, stay small against its
// K/V), so that the grid holds about kPrefillSplitTarget workgroups, and
// merges the pieces' partial states by log-sum-exp.  bytes: the workspace it
// needs (0: no split).
constexpr int64_t kPrefillSplitBelow = 512;
// Prefill workgroups rank the sequences by context length (longest first) up
// to this many sequences (one per thread of a workgroup; every workgroup
// pays a comparison per sequence, and the workgroups grow with the batch:
// at 256 sequences the ranking cost the fp16 MHA launch 15%).
constexpr int32_t kPrefillRankMax = 128;
constexpr int64_t kPrefillSplitTarget = 2048;
constexpr int32_t kPrefillMinSplitTiles = 32;
struct PrefillSplit {
  int32_t column_blocks = 1, rows_per_seq = 0, split_tiles = 0, split_max = 1;
  size_t ml_bytes = 0, bytes = 0;
};
inline PrefillSplit prefill_split(int32_t group, int32_t max_query_len, int32_t max_context_len, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  PrefillSplit p;
  p.column_blocks = prefill_column_blocks(group, max_query_len, num_seqs, num_kv_heads);
  const int64_t tpw = 4 * p.column_blocks * (16 / group);
  const int64_t qblocks = (int64_t(max_query_len) + tpw - 1) / tpw;
  p.rows_per_seq = static_cast<int32_t>(qblocks * tpw);
  const int64_t wgs = qblocks * num_seqs * num_kv_heads;
  const int64_t max_tiles = (int64_t(max_context_len) + 15) / 16;
  if (wgs <= 0 || wgs >= kPrefillSplitBelow || max_context_len <= 1) return p;
  const int64_t pieces = (kPrefillSplitTarget + wgs - 1) / wgs;
  int64_t spl = (max_tiles + pieces - 1) / pieces;
  spl = std::max<int64_t>(kPrefillMinSplitTiles, (spl + 1) & ~int64_t(1));
  // the chunk's first position is at most max_context_len - 1
  const int64_t smax = (int64_t(max_context_len) - 1) / (16 * spl) + 1;
  if (smax <= 1 || smax > 65535) return p;
  p.split_tiles = static_cast<int32_t>(spl);
  p.split_max = static_cast<int32_t>(smax);
  const size_t parts = size_t(smax) * size_t(num_seqs) * size_t(p.rows_per_seq) * size_t(num_q_heads);
  p.ml_bytes = (parts * 2 * sizeof(float) + 255) & ~size_t(255);
  p.bytes = p.ml_bytes + parts * size_t(head_dim) * sizeof(float);
  return p;
}

// launch_prefill with a context split (sp.split_tiles 0: none)
hipError_t launch_prefill_split(const PrefillArgs& a, const PrefillSplitArgs& sp, int32_t dtype, int32_t d,
                                int32_t bs, int32_t group, int32_t max_query_len, hipStream_t stream);

}  // namespace pa
