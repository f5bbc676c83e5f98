/*
 * pa.h — paged-attention decode on AMD MI355X (gfx950): C ABI of libpa.so.
 *
 * The library keeps a transformer's key/value cache in fixed-size blocks of
 * BS tokens that may sit anywhere in device memory, describes each sequence
 * by a block table (an ordered list of physical block ids) and runs
 * single-query decode attention that follows the table.  The idea and its
 * parts are those of the pages:
 *   [VM]  "Paged Attention: Virtual Memory for the KV Cache" (projectcozy.me)
 *   [MM]  "Paged Attention as a Memory Manager" (diomgis.com)
 *   [GL]  AI/ML term glossary, "Paged attention" (interviewkickstart.com)
 *
 * Conventions for every call
 *   - Device pointers are caller-owned device memory (e.g. torch tensors),
 *     contiguous, in the layouts stated below.  The library never allocates,
 *     frees or synchronises device memory; work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and returns immediately.
 *   - Host pointers are read or written before the call returns.
 *   - Every call returns a pa_status.  No C++ exception crosses the ABI.  On a
 *     non-OK status pa_last_error() returns a thread-local message.  Host
 *     arguments (sizes, dtypes, supported shapes) are validated before any
 *     launch; a failed launch maps to PA_ERR_HIP.
 *   - Device *contents* (table entries, slots, context lengths, copy pairs)
 *     are trusted like memcpy arguments: out-of-range ids or duplicate slots
 *     are undefined behaviour.  pa_check_tables() validates host copies.
 *   - Kernels are reentrant.  A block manager (pa_bm) is not thread-safe.
 *
 * Cache layout (one pool for K, one for V, per attention layer).  Both are
 * head-major inside a block, so the tile of one (block, kv head) is one
 * contiguous run of BS*D elements that a gather reads in full:
 *   K pool  [num_blocks][num_kv_heads][D / X][BS][X]   X = 16 / element bytes
 *           (8 for f16/bf16, 4 for f32): 16-byte chunks of a key, token-minor
 *   V pool  [num_blocks][num_kv_heads][D][BS]           tokens innermost
 * A slot s addresses token offset s % BS of block s / BS.
 *
 * Supported shapes: head_dim D in {64, 128}; block_size BS in {8, 16, 32};
 * num_q_heads % num_kv_heads == 0 with group g = num_q_heads / num_kv_heads
 * in {1, 2, 4, 8, 16}; num_blocks * BS < 2^31; element types below.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,      /* bad argument or unknown / duplicate sequence */
  PA_ERR_OOM = 2,          /* not enough free blocks; nothing was changed */
  PA_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed */
  PA_ERR_UNSUPPORTED = 4   /* valid but unsupported shape or dtype */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Decode kernel selection (pa_decode_variant).
 *   STREAM  matrix cores, every wave takes an equal share of all (sequence,
 *           kv head) tiles, direct global->LDS tile loads; 16-bit caches
 *   MFMA    matrix cores, one workgroup per (sequence, kv head, partition);
 *           16-bit caches
 *   VALU    vector ALU, one workgroup per (sequence, kv head, head group,
 *           partition); every dtype
 * AUTO picks STREAM for 16-bit caches and VALU for fp32. */
typedef enum {
  PA_KERNEL_AUTO = 0,
  PA_KERNEL_VALU = 1,
  PA_KERNEL_MFMA = 2,
  PA_KERNEL_STREAM = 3
} pa_kernel;

const char* pa_last_error(void);
const char* pa_version(void);

/* ------------------------------------------------------------------------
 * pa_write_kv — write the keys and values of num_tokens tokens into their
 * slots.  A request fills the block it holds before it asks for another
 * ([VM] §The fix borrowed from operating systems); the slots come from the
 * block manager.
 *   k_cache, v_cache   device pools in the layout above (written)
 *   k_new, v_new       device [num_tokens][num_kv_heads][head_dim], dtype
 *   slot_mapping       device int32 [num_tokens]; slot < 0 skips the token
 *                      (lets callers pad a batch).  Slots of one call must be
 *                      distinct and < num_blocks * block_size.
 * Errors: PA_ERR_INVALID for negative sizes or a non-16-byte-multiple row;
 * PA_ERR_UNSUPPORTED for shapes outside the supported set.  num_tokens = 0 is
 * a no-op.
 * ---------------------------------------------------------------------- */
pa_status pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                      void* stream);

/* ------------------------------------------------------------------------
 * pa_copy_blocks — whole-block copies for copy-on-write: a sequence about to
 * write into a block it shares gets its own copy first ([VM] §Sharing comes
 * almost for free; [MM] §Virtual Memory as the Blueprint).  For each pair
 * (src, dst) the K and V tiles of every kv head of block dst become a byte
 * copy of block src (all BS slots, written or not).
 *   pairs   device int32 [num_pairs][2] = (src, dst); destinations distinct
 *           and never a source of the same call.
 * Errors as pa_write_kv.  num_pairs = 0 is a no-op.  Issue it before the
 * pa_write_kv of the same step on the same stream.
 * ---------------------------------------------------------------------- */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode — one query token per sequence attends over its whole context
 * through its block table: the kernel follows the table instead of assuming
 * the sequence is laid out end to end ([VM] §The fix borrowed from operating
 * systems; [GL] "What is Paged Attention?"), so the result is plain softmax
 * attention over the logical sequence:
 *     out[i][r] = sum_t softmax_t(scale * q[i][r] . K_i[t][r / g]) V_i[t][r / g]
 * for t < context_lens[i]; query heads [h*g, (h+1)*g) share kv head h
 * (grouped-query attention, [VM] §What it does not fix).  A zero context
 * gives a zero row.  Softmax runs with a running maximum in fp32, products
 * accumulate in fp32.
 *   out            device [num_seqs][num_q_heads][head_dim], out_dtype = PA_F32
 *                  or kv_dtype (then rounded to nearest even from fp32)
 *   q              device [num_seqs][num_q_heads][head_dim], kv_dtype
 *   block_tables   device int32 [num_seqs][table_stride]; entry j is the
 *                  physical block of logical block j; entries past
 *                  ceil(ctx/BS) are never read
 *   context_lens   device int32 [num_seqs], 0 <= ctx <= max_context_len and
 *                  ceil(ctx/BS) <= table_stride
 *   max_context_len host-known upper bound of context_lens; it sizes the grid
 *   partition_size  tokens per work item (split-K); a multiple of 64 and of
 *                  4*BS, or 0 to let the library choose.  Sequences longer
 *                  than one partition are reduced in two passes: per-
 *                  partition partials (max, sum, unnormalised output) then a
 *                  log-sum-exp merge.
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...)
 *                  bytes for the same num_seqs/num_q_heads/num_kv_heads/
 *                  head_dim/max_context_len/partition_size (any contents;
 *                  256-byte aligned).  Calls that share one workspace must
 *                  be ordered (one stream).
 * Errors: PA_ERR_INVALID (bad sizes, workspace too small, out_dtype not F32
 * or kv_dtype), PA_ERR_UNSUPPORTED (shape outside the supported set),
 * PA_ERR_HIP (launch failure).
 * Cache policy: with a 16-bit cache the K/V tiles are read with the
 * non-temporal load policy (a byte is read once per call).  A block that
 * several sequences of the call share is then fetched once per sharer;
 * pa_step, which knows the refcounts, keeps the caching policy for those.
 * Results do not depend on the policy.
 * ---------------------------------------------------------------------- */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size);

/* The partition size pa_decode uses when passed 0 for these arguments. */
int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t max_context_len, int32_t block_size);

pa_status pa_decode(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                    const void* v_cache, pa_dtype kv_dtype, const int32_t* block_tables,
                    int32_t table_stride, const int32_t* context_lens, int32_t max_context_len,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments without the workspace, the same
 * kernels (automatic selection) and results.  The workspace is a static
 * array of PA_DECODE_SCRATCH_BYTES in device memory, one per device, set up
 * on the first call on that device and held until the process ends; the call
 * itself allocates nothing.  Its contents need no clearing (every byte a
 * call reads, the same call wrote first).  Every call on one device shares
 * that device's array: calls that may overlap on one device (different
 * streams, or host threads) race and must be ordered by the caller.
 * Errors: those of pa_decode; PA_ERR_INVALID when the call needs more
 * workspace than the array holds (every stream-kernel shape fits; partition
 * kernels need B x Hq x ceil(max_ctx / partition) x (D + 2) x 4 bytes);
 * PA_ERR_HIP when the array's device address cannot be obtained.
 * ---------------------------------------------------------------------- */
#define PA_DECODE_SCRATCH_BYTES (32u << 20)

pa_status pa_decode_noalloc(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                            const void* v_cache, pa_dtype kv_dtype, const int32_t* block_tables,
                            int32_t table_stride, const int32_t* context_lens, int32_t max_context_len,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                            void* stream);

/* pa_decode with an explicit kernel choice (for measurement): PA_KERNEL_VALU
 * supports every shape above; PA_KERNEL_MFMA and PA_KERNEL_STREAM need a
 * 16-bit kv_dtype (STREAM ignores partition_size). */
pa_status pa_decode_variant(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                            const void* v_cache, pa_dtype kv_dtype, const int32_t* block_tables,
                            int32_t table_stride, const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, void* stream,
                            pa_kernel kernel);

/* pa_decode in its two phases, for callers that time or schedule them apart:
 * phase 1 is the pass over the K/V tiles (it writes every output row that one
 * work item covers and the partial (max, sum, unnormalised output) of the
 * others), phase 2 the log-sum-exp merge of those partials; phase 3 runs both
 * (= pa_decode_variant).  Phase 2 must follow phase 1 of the same arguments
 * and workspace on the same stream. */
typedef enum { PA_PHASE_PASS = 1, PA_PHASE_MERGE = 2, PA_PHASE_ALL = 3 } pa_phase;

pa_status pa_decode_phase(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                          const void* v_cache, pa_dtype kv_dtype, const int32_t* block_tables,
                          int32_t table_stride, const int32_t* context_lens, int32_t max_context_len,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                          void* workspace, size_t workspace_bytes, void* stream, pa_kernel kernel,
                          int32_t phase);

/* ------------------------------------------------------------------------
 * Host block manager: the shared pool of interchangeable blocks, per-block
 * sharer counts and per-sequence block tables ([VM] §The fix borrowed from
 * operating systems, §Sharing comes almost for free; [MM] §How the Kernel
 * Executes Paged Attention; [GL] "What is Paged Attention?").
 *
 * Policy (the pages leave it open; it is fixed so results are unique):
 *   - the free list is a LIFO stack; pa_bm_create stacks it so the first
 *     allocation returns initial_order[0] (0,1,2,... when NULL);
 *   - add_seq(n) takes ceil(n/BS) blocks in logical order;
 *     slot(t) = table[t / BS] * BS + t % BS;
 *   - an append at position pos takes a new block when pos % BS == 0;
 *     otherwise, if the last block is shared (count > 1), it takes a new
 *     block, lowers the old block's count, points the table at the new block
 *     and reports the pair (old, new) for pa_copy_blocks; the last remaining
 *     sharer writes in place.  A batch is applied in list order;
 *   - fork copies the parent's table and raises each block's count;
 *   - free_seq lowers counts in logical order and pushes each block whose
 *     count reaches zero at once.
 * Every call is all-or-nothing: PA_ERR_OOM and PA_ERR_INVALID leave the
 * manager unchanged.  Sequence ids are arbitrary int64 keys.
 * ---------------------------------------------------------------------- */
typedef struct pa_bm pa_bm;

/* NULL on invalid arguments (see pa_last_error): num_blocks < 0, block_size
 * <= 0, or initial_order not a permutation of 0..num_blocks-1. */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order);
void pa_bm_destroy(pa_bm* bm);

/* New sequence holding num_tokens tokens; slots_out (host, [num_tokens], may
 * be NULL) receives their slots.  INVALID if seq exists or num_tokens < 0. */
pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq, int32_t num_tokens, int32_t* slots_out);

/* One new token for each of seqs[0..n): slots_out[n] receives its slot,
 * cow_pairs_out[n][2] the (src, dst) block copies to run first (host
 * buffers), *num_cow_out their count.  INVALID for unknown or repeated ids. */
pa_status pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* slots_out,
                             int32_t* cow_pairs_out, int32_t* num_cow_out);

pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);
pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq);

/* tables_out host int32 [n][stride] padded with -1; ctx_lens_out host int32
 * [n].  INVALID if a table is longer than stride or an id is unknown. */
pa_status pa_bm_export(const pa_bm* bm, const int64_t* seqs, int32_t n, int32_t stride,
                       int32_t* tables_out, int32_t* ctx_lens_out);

/* Free blocks: the headroom a server can admit against ([VM] §What it buys
 * in practice). */
int32_t pa_bm_num_free(const pa_bm* bm);
/* Preemption by swap ([VM] §What it does not fix: when memory runs out a
 * sequence is evicted and its blocks swapped out, to be brought back later).
 * pa_bm_swap_out releases the sequence's blocks like pa_bm_free_seq and keeps
 * its length: blocks_out (room for ceil(len / BS)) receives its table in
 * logical order and *num_blocks_out the count, so the caller can copy them
 * out (pa_swap_blocks, to_host = 1) on the stream before anything reuses
 * them.  A shared block stays resident for its other sharers; the swapped
 * sequence gets a private copy back.
 * pa_bm_swap_in gives a swapped-out sequence fresh blocks (all-or-nothing,
 * PA_ERR_OOM leaves everything unchanged) and returns them in logical order
 * for the copy back (to_host = 0).  pa_bm_swapped_len is the length of a
 * swapped-out sequence, or -1. */
pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq, int32_t* blocks_out, int32_t* num_blocks_out);
pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq, int32_t* blocks_out, int32_t* num_blocks_out);
int32_t pa_bm_swapped_len(const pa_bm* bm, int64_t seq);

/* Prefix caching across requests ([VM] §Sharing comes almost for free and
 * §Why this matters: a prompt prefix many requests share is stored once).
 * pa_bm_add_seq_cached is pa_bm_add_seq for a prompt given by its token ids
 * (tokens host int32 [num_tokens]): it walks the prompt's full blocks from the
 * start and reuses every cached block found, stopping at the first miss and
 * never reusing the block that holds the last token.  slots_out (room for
 * num_tokens, or NULL) gets every token's slot; *cached_tokens_out the number
 * of leading tokens whose K/V is already in the pool (a multiple of the block
 * size): the caller writes K/V and runs prefill for the rest only.  Its other
 * full blocks are cached at once under the key (content id of the previous
 * block, the block's token ids), compared exactly; their K/V must be written
 * on the stream before any later work reads them.
 * A cached block whose last reference goes is kept, evictable, instead of
 * freed; a sequence's blocks become evictable from its last to its first.
 * Fresh blocks come from the free stack, then from the evictable blocks,
 * oldest first (an evicted block's key is dropped).  pa_bm_num_free,
 * pa_bm_admit and out[0] of pa_bm_stats count the evictable blocks as free;
 * pa_bm_free_list lists the free stack only.  All-or-nothing: PA_ERR_OOM
 * changes nothing. */
pa_status pa_bm_add_seq_cached(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                               int32_t* slots_out, int32_t* cached_tokens_out);
/* out[4] = {cached blocks, evictable blocks, blocks reused so far, full blocks
 * looked up so far} */
pa_status pa_bm_cache_stats(const pa_bm* bm, int64_t* out);
/* Forget every cached prefix: evictable blocks go on the free stack (oldest
 * first), live cached blocks become plain blocks. */
pa_status pa_bm_cache_clear(pa_bm* bm);

/* Admission that keeps headroom ([VM] §What it buys in practice: memory is
 * handed out in small increments, so a server can admit without committing to
 * a request's worst case and can tell how close it is to the ceiling):
 * pa_bm_add_seq only if the blocks of num_tokens plus reserve_blocks (room the
 * caller keeps for the growth of live sequences) are free; else PA_ERR_OOM
 * and nothing changes. */
pa_status pa_bm_admit(pa_bm* bm, int64_t seq, int32_t num_tokens, int32_t reserve_blocks, int32_t* slots_out);
/* Occupancy in token slots ([VM] §The fix borrowed from operating systems:
 * at most one partly filled block per request):
 * out[4] = {slots of the blocks held (shared blocks once), tokens of all
 * sequences (shared tokens once per sequence), unused slots in the sequences'
 * last blocks, free slots}. */
pa_status pa_bm_occupancy(const pa_bm* bm, int64_t* out);
int32_t pa_bm_refcount(const pa_bm* bm, int32_t block);      /* -1 if out of range */
int32_t pa_bm_seq_len(const pa_bm* bm, int64_t seq);         /* -1 if unknown */
/* Blocks at the front of the sequence's table that are also held elsewhere
 * (refcount above one: a fork, a sharer not yet diverged, a cached prefix
 * another prompt reuses); -1 if unknown.  Kept per sequence and walked again
 * only after some block starts or stops being shared ([VM] §Sharing comes
 * almost for free).  pa_step records it for the decode pass's load policy. */
int32_t pa_bm_shared_blocks(const pa_bm* bm, int64_t seq);
int32_t pa_bm_num_seqs(const pa_bm* bm);
/* Free list, next allocation first; writes min(cap, num_free) ids, returns
 * num_free. */
int32_t pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap);
/* out[5] = {free blocks, referenced blocks, shared blocks (count > 1),
 *           copy-on-write pairs issued so far, slack tokens in last blocks} */
pa_status pa_bm_stats(const pa_bm* bm, int64_t* out);

/* Copies whole blocks (every kv head, K and V) between the pools and host
 * memory for preemption by swap: blocks[i] (pool block id) <-> slot i of
 * host_k / host_v, each [num_blocks_moved][num_kv_heads * head_dim *
 * block_size] elements in the pools' in-block layout.  to_host: 1 pool ->
 * host, 0 host -> pool.  host_k, host_v and blocks must be pinned host memory
 * (or device memory); 16-byte aligned buffers.  An id outside
 * [0, num_blocks) moves nothing (its host slot is left as it was).
 * Asynchronous on `stream`: the copy out must be enqueued before any work
 * that reuses the blocks, and the host must not read host_k / host_v before
 * it completes. */
pa_status pa_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v, const int32_t* blocks,
                         int32_t num_blocks_moved, int32_t to_host, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_prefill — causal attention of new tokens over their sequences' paged
 * context, the step before decode ([MM] §How the Kernel Executes Paged
 * Attention; [VM] §The fix borrowed from operating systems).
 * Sequence i's chunk is the query rows query_start[i] .. query_start[i+1] - 1
 * of q ([T][num_q_heads][head_dim], kv dtype, T = query_start[num_seqs]);
 * its context_lens[i] tokens (the chunk's own last, their K/V written through
 * the slots before this call) are read through block_tables like pa_decode.
 * Row t of a chunk of L tokens sits at position context_lens[i] - L + t and
 * attends to positions 0 .. itself (textbook causal attention; the pages give
 * no formula):
 *   out[row][h] = softmax_j(scale * q[row][h] . K[j][h / g]) V[j][h / g],
 *   j = 0 .. position.
 * out: [T][num_q_heads][head_dim] in F32 or the kv dtype.  query_start and
 * context_lens are device arrays; max_query_len (>= every chunk length) and
 * max_context_len (>= every context length, <= table_stride * block_size)
 * are host bounds that size the grid; device lengths are clamped to them.
 * 16-bit caches only (PA_ERR_UNSUPPORTED for F32); group in {1,2,4,8,16};
 * at most 65535 (sequence, kv head) pairs.
 * workspace (device, 16-byte aligned, caller-owned, any contents; may be
 * NULL): with it, a launch of few workgroups (short chunks, where one
 * workgroup would stream a whole context) splits each sequence's prefix
 * into pieces and merges their partial states by log-sum-exp (the same
 * softmax, summed in another order); it must then hold
 * pa_prefill_workspace_bytes(...) bytes (PA_ERR_INVALID if smaller).  NULL,
 * or a shape the library does not split, streams each context in one piece.
 * Asynchronous on `stream`.
 * ---------------------------------------------------------------------- */
pa_status pa_prefill(void* out, pa_dtype out_dtype, const void* q, const void* k_cache, const void* v_cache,
                     pa_dtype kv_dtype, const int32_t* block_tables, int32_t table_stride,
                     const int32_t* query_start, const int32_t* context_lens, int32_t max_query_len,
                     int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Workspace bytes pa_prefill's context split needs for a launch of this
 * shape (same bounds as the call); 0 when the library streams each context
 * in one piece (or the shape is invalid). */
size_t pa_prefill_workspace_bytes(int32_t max_query_len, int32_t max_context_len, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);

/* Column blocks per wave pa_prefill takes for a launch of this shape (each
 * wave holds CB blocks of 16 query columns, (16 / group) tokens each, so a
 * workgroup covers 64 CB / group query tokens): 3 when that leaves at least
 * 1024 workgroups and rounding max_query_len up to whole query blocks pads at
 * most a fifth of the rounded rows, 2 when that leaves at least 512 and the
 * padding is at most a fifth, else 1 (a chunk shorter than one block of a
 * count takes neither); 0 for a group size pa_prefill rejects.
 * For callers that count what a launch streams. */
int32_t pa_prefill_column_blocks(int32_t num_q_heads, int32_t num_kv_heads, int32_t max_query_len, int32_t num_seqs);

/* ------------------------------------------------------------------------
 * pa_step — one decode step of a batch, host and device parts in one call:
 *   1. pa_bm_append_slots: the new token of each of seqs[0..n) gets a slot
 *      (a fresh block when the last one is full; a copy of a shared last
 *      block first, [VM] §Sharing comes almost for free);
 *   2. pa_bm_export of the grown tables and context lengths;
 *   3. the step record, laid out in int32 words as
 *      [slots n | copy pairs 2n | context lengths n | tables n * table_stride
 *       | tile prefix sums n + 1 | shared blocks n | header 4
 *       | stream plan (16-byte aligned)]
 *      (shared blocks: how many blocks at the front of each table other
 *      sequences also hold, i.e. have a refcount above one; the stream pass
 *      reads their tiles with the caching load policy, every other K/V tile
 *      with the non-temporal one; the header: copy-on-write pairs, the
 *      stream grid of the plan or 0, cut items, words in use)
 *      (rounded up to a multiple of 4 words), goes from stage_host (pinned
 *      host memory, 16-byte aligned) to stage_dev (device memory): when the
 *      runtime maps stage_host into the device's address space, a kernel on
 *      the stream copies it and writes the new tokens in the same launch,
 *      otherwise a host-to-device copy precedes pa_write_kv.  The stream
 *      plan (16-bit caches, stream kernel selected) is the host's split of
 *      the (sequence, kv head, 16-token tile) list over the kernel's waves:
 *      each wave's first tile, then the items cut between waves with the
 *      waves holding them, so that the merge runs over cut items only;
 *   4. pa_copy_blocks of the copy pairs and the KV write of k_new/v_new
 *      ([n][num_kv_heads][head_dim], device) into the new slots;
 *   5. pa_decode_phase PASS then MERGE of q ([n][num_q_heads][head_dim])
 *      into out over the exported tables; pass_begin / pass_end (hipEvent_t
 *      or NULL) are recorded on the stream around the pass.
 * Everything is enqueued on `stream`.  stage_host must not be rewritten until
 * this call's kernels have read it (keep a ring of records guarded by
 * events); both stage buffers hold stage_words >= pa_step_record_words(n,
 * table_stride, num_kv_heads) int32 words.
 * *max_ctx_out (may be NULL) receives the longest context.  Errors leave the
 * manager unchanged and launch nothing: the decode arguments, the record
 * size and the stride (a sequence whose next token would not fit
 * table_stride blocks) are checked before any change.
 * Stream kernel only: wg_weights (host, num_weights =
 * pa_decode_stream_grid(...) entries, or NULL for equal shares) sets each
 * workgroup's share of the tiles (clamped to 1..65536).  The weights decide
 * where items are cut between waves, and so the order in which an item's
 * terms are summed and merged: results with different weights agree to fp32
 * rounding, not bit for bit; the same weights and lengths give the same bits.
 * wave_times (pinned host or device memory, 8 * grid int32, or
 * NULL) receives, for the 4 waves of each workgroup in order, the start and
 * end of the wave as the low 32 bits of the GPU's 100 MHz real-time counter
 * (compare stamps by signed difference), from which a caller can give slow
 * compute units smaller shares on later steps (written only when the stream
 * kernel runs).
 * ---------------------------------------------------------------------- */
pa_status pa_step(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* stage_host, int32_t* stage_dev,
                  size_t stage_words, int32_t table_stride, void* k_cache, void* v_cache, const void* k_new,
                  const void* v_new, const void* q, void* out, pa_dtype out_dtype, pa_dtype kv_dtype,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                  pa_kernel kernel, void* stream, void* pass_begin, void* pass_end, int32_t* max_ctx_out,
                  const int32_t* wg_weights, int32_t num_weights, int32_t* wave_times);

/* The device part of a step again, on the record the last pa_step left in
 * stage_host / stage_dev (neither rewritten since), for another layer of the
 * same model: its own pools, k_new / v_new, q and out, the same sequences,
 * slots, tables and plan (every layer of a decoder shares them).  phases:
 * bit 0 the copy-on-write copies and the KV write, bit 1 the decode pass,
 * bit 2 the merge (7 = the whole layer; a pass alone leaves `out` unfinished
 * for cut items until its merge runs).  Shapes and kernel must be those of
 * the pa_step call (checked against the record's header: INVALID
 * otherwise); pass_begin / pass_end / wave_times as in pa_step. */
pa_status pa_step_layer(const int32_t* stage_host, int32_t* stage_dev, int32_t n, int32_t table_stride,
                        void* k_cache, void* v_cache, const void* k_new, const void* v_new, const void* q, void* out,
                        pa_dtype out_dtype, pa_dtype kv_dtype, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                        void* workspace, size_t workspace_bytes, pa_kernel kernel, void* stream, int32_t phases,
                        void* pass_begin, void* pass_end, int32_t* wave_times);

/* Load-balance feedback for pa_step's wg_weights, from the wave_times of a
 * completed stream pass: out[c] (host, `classes` entries) receives the mean
 * finish time of the workgroups b with b % classes == c, a workgroup
 * finishing at the last end stamp of its four waves, counted from the
 * earliest start stamp of the pass (signed 32-bit differences of the
 * 100 MHz counter, in its ticks).  Workgroups are dealt to the GPU's dies in
 * turn, so with classes = 8 these are the dies' finish times.  INVALID for
 * null pointers or non-positive sizes. */
pa_status pa_stream_class_finish(const int32_t* wave_times, int32_t grid, int32_t classes, double* out);

/* Int32 words of a pa_step record for up to max_seqs sequences (0 for bad
 * sizes). */
size_t pa_step_record_words(int32_t max_seqs, int32_t table_stride, int32_t num_kv_heads);

/* The stream plan pa_step writes into its record, computed on the host for
 * inspection: tile_prefix[n + 1] (tiles of 16 tokens of the sequences before
 * each one; non-decreasing from 0), `grid` workgroups (1..1024) with weights
 * (NULL = equal).  Writes into out (out_words >= E + 8 n num_kv_heads +
 * 8 grid, E = 4 grid + 1 rounded up to a multiple of 4): the first tile of
 * each of the 4 grid waves and the end; from word E on, one 8-word entry per
 * item whose tiles fall to more than one wave, {2 * (seq * num_kv_heads +
 * kvh) + 1 when the item's first wave starts before it, its number of waves,
 * the offset of the first in the wave list, the first four waves (0 past the
 * count), 0}; then the wave list (every cut item's waves, in order).
 * *num_cut receives the entries.  Returns the words written, or -1 for bad
 * arguments. */
int64_t pa_stream_plan(const int32_t* tile_prefix, int32_t n, int32_t num_kv_heads, int32_t grid,
                       const int32_t* weights, int32_t* out, size_t out_words, int32_t* num_cut);

/* Workgroups of the stream kernel for this shape (0 when pa_decode would not
 * use it): the length of pa_step's wg_weights. */
int32_t pa_decode_stream_grid(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim);

/* Debug validator over HOST copies of the decode inputs: every table entry a
 * sequence reads is in [0, num_blocks) and ceil(ctx/BS) <= stride.  Returns
 * INVALID with the first offending (sequence, entry) in pa_last_error(). */
pa_status pa_check_tables(const int32_t* tables, int32_t n, int32_t stride,
                          const int32_t* ctx_lens, int32_t block_size, int32_t num_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
