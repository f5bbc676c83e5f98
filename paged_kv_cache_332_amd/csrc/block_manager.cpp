// Host block manager: shared free list of interchangeable fixed-size blocks,
// per-block sharer counts and per-sequence block tables.
//
// From the pages: blocks are handed out one at a time when the last one is
// full and returned to a shared pool the moment a request finishes
// ("Paged Attention: Virtual Memory for the KV Cache", §The fix borrowed from
// operating systems; glossary "What is Paged Attention?"); prefill numbers
// logical blocks in order and takes physical blocks from a free list
// ("Paged Attention as a Memory Manager", §How the Kernel Executes Paged
// Attention); tables of block references can share a block, and a sharer that
// diverges copies the block it is about to write (§Sharing comes almost for
// free).  The allocation policy the pages leave open is stated in pa.h.
#include <algorithm>
#include <cstring>
#include <iterator>
#include <list>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

// A cached full block is named by the content id of the block before it (0 for
// a prompt's first block) and its own token ids: the key names the whole
// prefix up to the block's end, and lookups compare it exactly.
struct PrefixKey {
  uint64_t parent = 0;
  std::vector<int32_t> tokens;
  bool operator==(const PrefixKey& o) const { return parent == o.parent && tokens == o.tokens; }
};
// Bucket hash only (FNV-1a, 64 bit, over the parent id and the token bytes).
struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const {
    uint64_t h = 14695981039346656037ull;
    auto mix = [&h](const void* p, size_t n) {
      const unsigned char* c = static_cast<const unsigned char*>(p);
      for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 1099511628211ull;
    };
    mix(&k.parent, sizeof(k.parent));
    mix(k.tokens.data(), k.tokens.size() * sizeof(int32_t));
    return static_cast<size_t>(h);
  }
};

struct pa_bm {
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
    // blocks at the front of the table with refcount > 1, valid while
    // shared_epoch equals the manager's share_epoch
    mutable int32_t shared_len = 0;
    mutable uint64_t shared_epoch = 0;
    uint64_t batch_mark = 0;  // the append batch that last listed this sequence
  };
  struct CacheEntry {
    uint64_t cid;
    int32_t block;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 1;
  std::vector<int32_t> free_stack;  // back() is the next block handed out
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int64_t, int32_t> swapped;  // lengths of sequences held on the host
  int64_t cow_count = 0;
  // prefix cache
  std::unordered_map<PrefixKey, CacheEntry, PrefixKeyHash> cache;
  std::unordered_map<int32_t, PrefixKey> block_key;  // cached block -> its key
  std::list<int32_t> evictable;                      // cached, unreferenced; front = oldest
  std::unordered_map<int32_t, std::list<int32_t>::iterator> evictable_at;
  uint64_t next_cid = 1;
  int64_t hit_blocks = 0, query_blocks = 0;
  // advanced whenever a block starts or stops being shared (its refcount
  // crosses between 1 and 2), which can change any table's shared prefix
  uint64_t share_epoch = 1;
  // per-append-batch scratch: the count a last block will have once the
  // batch's earlier copies are done, valid where batch_rc_mark[b] equals
  // the batch number
  uint64_t batch = 0;
  std::vector<uint64_t> batch_rc_mark;
  std::vector<int32_t> batch_rc;
  std::vector<Seq*> batch_seqs;

  // refcount[b] += d, noting a change of the block's shared state
  void rc_add(int32_t b, int32_t d) {
    const int32_t before = refcount[b];
    refcount[b] = before + d;
    if ((before > 1) != (before + d > 1)) ++share_epoch;
  }
  // The number of blocks at the front of s's table that other holders share
  // (walked again only after a sharing change anywhere).
  int32_t shared_prefix(const Seq& s) const {
    if (s.shared_epoch != share_epoch) {
      int32_t j = 0;
      const int32_t nb = static_cast<int32_t>(s.table.size());
      while (j < nb && refcount[s.table[j]] > 1) ++j;
      s.shared_len = j;
      s.shared_epoch = share_epoch;
    }
    return s.shared_len;
  }

  // blocks a call can get: the free stack, then the evictable cached blocks
  int64_t available() const { return static_cast<int64_t>(free_stack.size() + evictable.size()); }
  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = evictable.front();
      evictable.pop_front();
      evictable_at.erase(b);
      auto k = block_key.find(b);
      cache.erase(k->second);
      block_key.erase(k);
    }
    refcount[b] = 1;
    return b;
  }
  // One reference of each block dropped in logical order; a block reaching
  // zero goes on the free stack or, if cached, to the evictable list (the
  // table's cached blocks from last to first, so a prefix's end goes first).
  void release(const std::vector<int32_t>& table) {
    std::vector<int32_t> cached;
    for (int32_t b : table) {
      rc_add(b, -1);
      if (refcount[b] == 0) {
        if (block_key.count(b)) cached.push_back(b);
        else free_stack.push_back(b);
      }
    }
    for (auto it = cached.rbegin(); it != cached.rend(); ++it) {
      evictable.push_back(*it);
      evictable_at[*it] = std::prev(evictable.end());
    }
  }
  int32_t slot(const Seq& s, int32_t pos) const {
    return s.table[pos / block_size] * block_size + pos % block_size;
  }
};

extern "C" {

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order) {
  if (num_blocks < 0 || block_size <= 0 ||
      static_cast<int64_t>(num_blocks) * block_size >= (int64_t(1) << 31)) {
    pa::fail(PA_ERR_INVALID, "pa_bm_create: bad num_blocks %d / block_size %d", num_blocks,
             block_size);
    return nullptr;
  }
  auto* bm = new pa_bm;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  bm->free_stack.resize(num_blocks);
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = initial_order ? initial_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      pa::fail(PA_ERR_INVALID, "pa_bm_create: initial_order is not a permutation (entry %d)", i);
      return nullptr;
    }
    seen[b] = 1;
    bm->free_stack[num_blocks - 1 - i] = b;  // order[0] ends on top
  }
  return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq, int32_t num_tokens, int32_t* slots_out) {
  if (!bm || num_tokens < 0) return pa::fail(PA_ERR_INVALID, "pa_bm_add_seq: bad arguments");
  if (bm->seqs.count(seq) || bm->swapped.count(seq))
    return pa::fail(PA_ERR_INVALID, "pa_bm_add_seq: sequence %lld exists", (long long)seq);
  int64_t need = (static_cast<int64_t>(num_tokens) + bm->block_size - 1) / bm->block_size;
  if (need > bm->available())
    return pa::fail(PA_ERR_OOM, "pa_bm_add_seq: need %lld blocks, %lld free", (long long)need,
                    (long long)bm->available());
  pa_bm::Seq s;
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->take());
  s.len = num_tokens;
  if (slots_out)
    for (int32_t t = 0; t < num_tokens; ++t) slots_out[t] = bm->slot(s, t);
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_bm_admit(pa_bm* bm, int64_t seq, int32_t num_tokens, int32_t reserve_blocks, int32_t* slots_out) {
  if (!bm || num_tokens < 0 || reserve_blocks < 0) return pa::fail(PA_ERR_INVALID, "pa_bm_admit: bad arguments");
  const int64_t need = (static_cast<int64_t>(num_tokens) + bm->block_size - 1) / bm->block_size;
  const int64_t free_blocks = bm->available();
  if (need + reserve_blocks > free_blocks)
    return pa::fail(PA_ERR_OOM, "pa_bm_admit: need %lld blocks and a reserve of %d, %lld free", (long long)need,
                    reserve_blocks, (long long)free_blocks);
  return pa_bm_add_seq(bm, seq, num_tokens, slots_out);
}

pa_status pa_bm_occupancy(const pa_bm* bm, int64_t* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID, "pa_bm_occupancy: bad arguments");
  int64_t held = 0, tokens = 0, slack = 0;
  for (int32_t c : bm->refcount) held += c > 0;
  for (const auto& kv : bm->seqs) {
    tokens += kv.second.len;
    slack += static_cast<int64_t>(kv.second.table.size()) * bm->block_size - kv.second.len;
  }
  out[0] = held * bm->block_size;
  out[1] = tokens;
  out[2] = slack;
  out[3] = bm->available() * bm->block_size;
  return PA_OK;
}

pa_status pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* slots_out,
                             int32_t* cow_pairs_out, int32_t* num_cow_out) {
  if (!bm || n < 0 || (n > 0 && (!seqs || !slots_out || !cow_pairs_out)) || !num_cow_out)
    return pa::fail(PA_ERR_INVALID, "pa_bm_append_slots: bad arguments");
  // Validate and count the fresh blocks first so the call is all-or-nothing.
  const uint64_t mark = ++bm->batch;
  if (bm->batch_rc_mark.size() != size_t(bm->num_blocks)) {
    bm->batch_rc_mark.assign(size_t(bm->num_blocks), 0);
    bm->batch_rc.assign(size_t(bm->num_blocks), 0);
  }
  std::vector<pa_bm::Seq*>& ptr = bm->batch_seqs;
  ptr.resize(size_t(n));
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return pa::fail(PA_ERR_INVALID, "pa_bm_append_slots: unknown sequence %lld", (long long)seqs[i]);
    if (it->second.batch_mark == mark)
      return pa::fail(PA_ERR_INVALID, "pa_bm_append_slots: sequence %lld repeated", (long long)seqs[i]);
    it->second.batch_mark = mark;
    ptr[i] = &it->second;
    const pa_bm::Seq& s = it->second;
    if (s.len % bm->block_size == 0) {
      ++need;
    } else {
      const int32_t last = s.table.back();
      if (bm->batch_rc_mark[last] != mark) {
        bm->batch_rc_mark[last] = mark;
        bm->batch_rc[last] = bm->refcount[last];
      }
      if (bm->batch_rc[last] > 1) {
        ++need;
        --bm->batch_rc[last];
      }
    }
  }
  if (need > bm->available())
    return pa::fail(PA_ERR_OOM, "pa_bm_append_slots: need %lld blocks, %lld free", (long long)need,
                    (long long)bm->available());
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    pa_bm::Seq& s = *ptr[i];
    int32_t pos = s.len;
    if (pos % bm->block_size == 0) {
      s.table.push_back(bm->take());
    } else if (bm->refcount[s.table.back()] > 1) {
      int32_t old = s.table.back();
      int32_t fresh = bm->take();
      bm->rc_add(old, -1);
      s.table.back() = fresh;
      // the copy is private: a cached shared prefix ends before it at most
      const int32_t at = static_cast<int32_t>(s.table.size()) - 1;
      if (s.shared_len > at) s.shared_len = at;
      cow_pairs_out[2 * ncow] = old;
      cow_pairs_out[2 * ncow + 1] = fresh;
      ++ncow;
    }
    slots_out[i] = bm->slot(s, pos);
    s.len = pos + 1;
  }
  bm->cow_count += ncow;
  *num_cow_out = ncow;
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return pa::fail(PA_ERR_INVALID, "pa_bm_fork: null manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || bm->seqs.count(child) || bm->swapped.count(child))
    return pa::fail(PA_ERR_INVALID, "pa_bm_fork: unknown parent %lld or existing child %lld",
                    (long long)parent, (long long)child);
  pa_bm::Seq s = it->second;
  for (int32_t b : s.table) bm->rc_add(b, 1);
  bm->seqs.emplace(child, std::move(s));
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq) {
  if (!bm) return pa::fail(PA_ERR_INVALID, "pa_bm_free_seq: null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end())
    return pa::fail(PA_ERR_INVALID, "pa_bm_free_seq: unknown sequence %lld", (long long)seq);
  for (int32_t b : it->second.table) {
    if (bm->refcount[b] <= 0)
      return pa::fail(PA_ERR_INVALID, "pa_bm_free_seq: refcount underflow on block %d", b);
  }
  bm->release(it->second.table);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq, int32_t* blocks_out, int32_t* num_blocks_out) {
  if (!bm || !num_blocks_out) return pa::fail(PA_ERR_INVALID, "pa_bm_swap_out: bad arguments");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end())
    return pa::fail(PA_ERR_INVALID, "pa_bm_swap_out: unknown sequence %lld", (long long)seq);
  const std::vector<int32_t>& t = it->second.table;
  if (!t.empty() && !blocks_out) return pa::fail(PA_ERR_INVALID, "pa_bm_swap_out: bad arguments");
  for (int32_t b : t) {
    if (bm->refcount[b] <= 0)
      return pa::fail(PA_ERR_INVALID, "pa_bm_swap_out: refcount underflow on block %d", b);
  }
  std::copy(t.begin(), t.end(), blocks_out);
  *num_blocks_out = static_cast<int32_t>(t.size());
  // released like pa_bm_free_seq: the caller copies the blocks out on the
  // same stream before anything can reuse them
  bm->release(t);
  bm->swapped[seq] = it->second.len;
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq, int32_t* blocks_out, int32_t* num_blocks_out) {
  if (!bm || !num_blocks_out) return pa::fail(PA_ERR_INVALID, "pa_bm_swap_in: bad arguments");
  auto it = bm->swapped.find(seq);
  if (it == bm->swapped.end() || bm->seqs.count(seq))
    return pa::fail(PA_ERR_INVALID, "pa_bm_swap_in: sequence %lld is not swapped out", (long long)seq);
  const int32_t len = it->second;
  const int64_t need = (static_cast<int64_t>(len) + bm->block_size - 1) / bm->block_size;
  if (need > 0 && !blocks_out) return pa::fail(PA_ERR_INVALID, "pa_bm_swap_in: bad arguments");
  if (need > bm->available())
    return pa::fail(PA_ERR_OOM, "pa_bm_swap_in: need %lld blocks, %lld free", (long long)need,
                    (long long)bm->available());
  pa_bm::Seq s;
  s.len = len;
  for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->take());
  std::copy(s.table.begin(), s.table.end(), blocks_out);
  *num_blocks_out = static_cast<int32_t>(need);
  bm->seqs.emplace(seq, std::move(s));
  bm->swapped.erase(it);
  return PA_OK;
}

pa_status pa_bm_add_seq_cached(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                               int32_t* slots_out, int32_t* cached_tokens_out) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !tokens) || !cached_tokens_out)
    return pa::fail(PA_ERR_INVALID, "pa_bm_add_seq_cached: bad arguments");
  if (bm->seqs.count(seq) || bm->swapped.count(seq))
    return pa::fail(PA_ERR_INVALID, "pa_bm_add_seq_cached: sequence %lld exists", (long long)seq);
  const int32_t BS = bm->block_size;
  const int64_t nb = (static_cast<int64_t>(num_tokens) + BS - 1) / BS;
  const int32_t full = num_tokens / BS;
  // the block holding the last token is always computed
  const int32_t lookable = num_tokens > 0 ? (num_tokens - 1) / BS : 0;
  PrefixKey key;
  key.tokens.resize(BS);
  uint64_t parent = 0;
  std::vector<int32_t> hits;
  int64_t revived = 0;
  for (int32_t i = 0; i < lookable; ++i) {
    key.parent = parent;
    std::memcpy(key.tokens.data(), tokens + static_cast<int64_t>(i) * BS, sizeof(int32_t) * BS);
    auto f = bm->cache.find(key);
    if (f == bm->cache.end()) break;
    parent = f->second.cid;
    hits.push_back(f->second.block);
    revived += bm->refcount[f->second.block] == 0;
  }
  const int64_t need = nb - static_cast<int64_t>(hits.size());
  if (need > bm->available() - revived)
    return pa::fail(PA_ERR_OOM, "pa_bm_add_seq_cached: need %lld blocks, %lld free", (long long)need,
                    (long long)(bm->available() - revived));
  bm->query_blocks += lookable;
  bm->hit_blocks += static_cast<int64_t>(hits.size());
  pa_bm::Seq s;
  s.len = num_tokens;
  s.table.reserve(nb);
  for (int32_t b : hits) {
    if (bm->refcount[b] == 0) {
      auto at = bm->evictable_at.find(b);
      bm->evictable.erase(at->second);
      bm->evictable_at.erase(at);
    }
    bm->rc_add(b, 1);
    s.table.push_back(b);
  }
  for (int64_t i = static_cast<int64_t>(hits.size()); i < nb; ++i) {
    const int32_t b = bm->take();
    s.table.push_back(b);
    if (i < full) {
      key.parent = parent;
      std::memcpy(key.tokens.data(), tokens + i * BS, sizeof(int32_t) * BS);
      auto f = bm->cache.find(key);
      if (f != bm->cache.end()) {
        parent = f->second.cid;  // already cached under another block: this one stays private
      } else {
        const uint64_t cid = bm->next_cid++;
        bm->cache.emplace(key, pa_bm::CacheEntry{cid, b});
        bm->block_key.emplace(b, key);
        parent = cid;
      }
    }
  }
  if (slots_out)
    for (int32_t t = 0; t < num_tokens; ++t) slots_out[t] = bm->slot(s, t);
  *cached_tokens_out = static_cast<int32_t>(hits.size()) * BS;
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_bm_cache_stats(const pa_bm* bm, int64_t* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID, "pa_bm_cache_stats: bad arguments");
  out[0] = static_cast<int64_t>(bm->block_key.size());
  out[1] = static_cast<int64_t>(bm->evictable.size());
  out[2] = bm->hit_blocks;
  out[3] = bm->query_blocks;
  return PA_OK;
}

pa_status pa_bm_cache_clear(pa_bm* bm) {
  if (!bm) return pa::fail(PA_ERR_INVALID, "pa_bm_cache_clear: null manager");
  for (int32_t b : bm->evictable) bm->free_stack.push_back(b);
  bm->evictable.clear();
  bm->evictable_at.clear();
  bm->cache.clear();
  bm->block_key.clear();
  return PA_OK;
}

int32_t pa_bm_swapped_len(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->swapped.find(seq);
  return it == bm->swapped.end() ? -1 : it->second;
}

pa_status pa_bm_export(const pa_bm* bm, const int64_t* seqs, int32_t n, int32_t stride,
                       int32_t* tables_out, int32_t* ctx_lens_out) {
  if (!bm || n < 0 || stride < 0 || (n > 0 && (!seqs || !tables_out || !ctx_lens_out)))
    return pa::fail(PA_ERR_INVALID, "pa_bm_export: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return pa::fail(PA_ERR_INVALID, "pa_bm_export: unknown sequence %lld", (long long)seqs[i]);
    if (static_cast<int64_t>(it->second.table.size()) > stride)
      return pa::fail(PA_ERR_INVALID, "pa_bm_export: sequence %lld holds %zu blocks > stride %d",
                      (long long)seqs[i], it->second.table.size(), stride);
  }
  for (int32_t i = 0; i < n; ++i) {
    const pa_bm::Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + static_cast<int64_t>(i) * stride;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + stride, -1);
    ctx_lens_out[i] = s.len;
  }
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_bm* bm) { return bm ? static_cast<int32_t>(bm->available()) : -1; }

int32_t pa_bm_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

int32_t pa_bm_seq_len(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pa_bm_shared_blocks(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : bm->shared_prefix(it->second);
}

int32_t pa_bm_num_seqs(const pa_bm* bm) { return bm ? static_cast<int32_t>(bm->seqs.size()) : -1; }

int32_t pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  int32_t nf = static_cast<int32_t>(bm->free_stack.size());
  for (int32_t i = 0; i < std::min(cap, nf); ++i) out[i] = bm->free_stack[nf - 1 - i];
  return nf;
}

pa_status pa_bm_stats(const pa_bm* bm, int64_t* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID, "pa_bm_stats: bad arguments");
  int64_t used = 0, shared = 0, waste = 0;
  for (int32_t c : bm->refcount) {
    used += c > 0;
    shared += c > 1;
  }
  for (const auto& kv : bm->seqs)
    waste += static_cast<int64_t>(kv.second.table.size()) * bm->block_size - kv.second.len;
  out[0] = bm->available();
  out[1] = used;
  out[2] = shared;
  out[3] = bm->cow_count;
  out[4] = waste;
  return PA_OK;
}

pa_status pa_check_tables(const int32_t* tables, int32_t n, int32_t stride, const int32_t* ctx_lens,
                          int32_t block_size, int32_t num_blocks) {
  if (n < 0 || stride < 0 || block_size <= 0 || (n > 0 && (!tables || !ctx_lens)))
    return pa::fail(PA_ERR_INVALID, "pa_check_tables: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    if (ctx_lens[i] < 0) return pa::fail(PA_ERR_INVALID, "pa_check_tables: ctx[%d] = %d < 0", i, ctx_lens[i]);
    int64_t nb = (static_cast<int64_t>(ctx_lens[i]) + block_size - 1) / block_size;
    if (nb > stride)
      return pa::fail(PA_ERR_INVALID, "pa_check_tables: sequence %d needs %lld entries > stride %d", i,
                      (long long)nb, stride);
    for (int64_t j = 0; j < nb; ++j) {
      int32_t b = tables[static_cast<int64_t>(i) * stride + j];
      if (b < 0 || b >= num_blocks)
        return pa::fail(PA_ERR_INVALID, "pa_check_tables: sequence %d entry %lld = %d out of [0, %d)", i,
                        (long long)j, b, num_blocks);
    }
  }
  return PA_OK;
}

}  // extern "C"
