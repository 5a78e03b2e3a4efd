/*
 * libpagedattn -- paged attention over a block-paged KV cache on MI355X (gfx950).
 *
 * The KV cache is cut into fixed-size blocks of block_size (B) tokens; each
 * sequence owns an append-only list of physical block ids (its block table),
 * and every attention call gathers K/V by walking that list in logical order.
 * ("PagedAttention: fragmentation, blocks, block tables", sections 1-3 and the
 * attention-metadata section; "The pantry of pigeonholes", "The mechanism";
 * "Memory management", Concept.)
 *
 * Conventions
 *   - Every call returns int status: PA_OK, PA_ERR_INVALID (bad argument, shape,
 *     pointer, id or duplicate), PA_ERR_NO_SPACE (the pool cannot supply the
 *     blocks: the allocate-returns-None case of the slot-allocation section),
 *     PA_ERR_HIP (a HIP launch failed) or PA_ERR_NO_MEMORY (the pool could
 *     not allocate host memory for its own bookkeeping; the pool is unchanged).  pa_last_error() describes the most
 *     recent failure on the calling thread.
 *   - Pool calls are all-or-nothing: on any error the pool is unchanged (CPU
 *     reference allocator section: a failed allocation leaves the sequence
 *     intact; "Memory management", Code: the capacity test precedes any change).
 *   - Ownership: the library owns the pool's host memory behind the opaque
 *     handle.  The caller owns every device buffer.  The library never
 *     allocates device memory; decode split-K scratch is a caller workspace
 *     sized by pa_paged_decode_workspace_size().
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as void*,
 *     NULL = the null stream) and never synchronize.  Argument errors are
 *     detected on the host before anything is enqueued.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 *
 * KV-cache layout (fixed)
 *   key_cache and value_cache are separate bf16 arrays.  Physical block b of a
 *   cache starts at element b * cache_block_stride and is laid out
 *   [B][num_kv_heads][head_dim] (token-major), so with
 *   cache_block_stride == B * num_kv_heads * head_dim the cache is the flat
 *   row-major [num_blocks * B][num_kv_heads][head_dim] array whose row s is
 *   slot s.  Block i then owns the contiguous range [i*page, (i+1)*page)
 *   (block-major storage, slot-mapping section).  A larger stride lets one
 *   allocation interleave several layers or K with V.
 *
 * Block tables are int32 [num_seqs][bt_stride]; row s lists sequence s's
 * physical blocks in logical order and only its first ceil(seq_lens[s] / B)
 * entries are read (attention-metadata section).  Entries past that may hold
 * anything.  Every entry that is read must lie in [0, num_blocks); kernels
 * clamp entries into that range so that a corrupt table cannot make them read
 * outside the cache (the result is then wrong, but no fault occurs).
 *
 * Supported kernel shapes: head_dim in {64, 128}; num_q_heads a multiple of
 * num_kv_heads with num_q_heads / num_kv_heads <= 8 (query head h reads KV
 * head h / (num_q_heads / num_kv_heads)); block_size a power of two in
 * [1, 256].  Anything else returns PA_ERR_INVALID.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,
  PA_ERR_NO_SPACE = -2,
  PA_ERR_HIP = -3,
  PA_ERR_NO_MEMORY = -4
};

/* Text of the most recent error on this thread ("" if none).  The pointer
 * stays valid until the next failing call on the same thread. */
const char* pa_last_error(void);

/* ------------------------------------------------------------------------ */
/* Host block pool (CPU only, not thread-safe: one pool per thread at a time) */
/* ------------------------------------------------------------------------ */

typedef struct pa_pool pa_pool;

/* Create a pool of num_blocks blocks of block_size tokens.  All blocks start
 * free with reference count 0, queued in ascending id order, or in the order
 * of initial_free_order (a permutation of 0..num_blocks-1) when it is not
 * NULL.  There is no reserved null block: every id is allocatable.
 * ("PagedAttention: fragmentation, blocks, block tables", 1. The block pool:
 * one metadata entry per physical block, all queued at construction.)
 * Errors: PA_ERR_INVALID for non-positive sizes, a non-permutation or a NULL
 * `out`. */
int pa_pool_create(int32_t num_blocks, int32_t block_size,
                   const int32_t* initial_free_order, pa_pool** out);

/* Destroy a pool (NULL is ignored). */
void pa_pool_destroy(pa_pool* pool);

/* Register a sequence with an empty block table.  Errors: PA_ERR_INVALID if
 * seq_id already exists. */
int pa_pool_add_seq(pa_pool* pool, int64_t seq_id);

/* Register a sequence whose prompt is tokens[0..n_tokens) and give it the
 * longest run of cached full blocks matching the prompt's leading blocks.
 * Block j's hash is 64-bit FNV-1a over the previous block's hash (8 bytes
 * little-endian; 0 before block 0) followed by the block's B token ids (4
 * bytes little-endian each), so a hash names the block's content at its
 * position.  Matching stops at the first full block whose hash is not cached;
 * a partial last block never matches.  Each hit block gains one reference and,
 * if it was free (cached but evictable), leaves the free queue.  The sequence
 * then holds hit_tokens = hits * B tokens whose KV is already in the cache; the
 * caller appends the rest of the prompt.
 * ("PagedAttention: fragmentation, blocks, block tables", 1. The block pool:
 * per-block hash and touch; copy-on-write section: a full-block prefix hit
 * needs no copy.  "The pantry of pigeonholes", prefix sharing: a block's hash
 * covers its tokens and its parent's hash.)
 * tokens: host int32 [n_tokens] (NULL allowed when n_tokens is 0).
 * Errors: PA_ERR_INVALID if seq_id exists or an argument is NULL/negative
 * (pool unchanged, *hit_tokens = 0). */
int pa_pool_add_seq_cached(pa_pool* pool, int64_t seq_id, const int32_t* tokens,
                           int64_t n_tokens, int64_t* hit_tokens);

/* Enter the full blocks of seq_id's first n_tokens tokens (whose KV the caller
 * has written) into the prefix cache: block j gets the chained hash of
 * tokens[0 .. (j+1)B).  A block that already holds that hash, or whose hash
 * another block already holds (the first block entered keeps it), is left as it
 * is.  All-or-nothing: if n_tokens exceeds the sequence's length or a block
 * already holds a different hash, PA_ERR_INVALID and nothing changes.
 * (Same passages as pa_pool_add_seq_cached.) */
int pa_pool_cache_blocks(pa_pool* pool, int64_t seq_id, const int32_t* tokens, int64_t n_tokens);

/* New sequence dst_seq shares every block of src_seq (same table, same
 * length); each shared block's reference count grows by one.  Full blocks are
 * then shared outright and a partial tail is copied on first write ("Memory
 * management", Maths; copy-on-write section: sharing by reference counts).
 * Errors: PA_ERR_INVALID if src_seq is unknown or dst_seq exists. */
int pa_pool_fork(pa_pool* pool, int64_t src_seq, int64_t dst_seq);

/* Append n_tokens >= 1 tokens to seq_id.
 *   needed = ceil((len + n) / B) - held;  copy = (len % B != 0) and the tail
 *   is shared (refcount > 1) or pinned by a transfer.  If needed + copy
 *   exceeds the free blocks, return PA_ERR_NO_SPACE and change nothing.
 *   Otherwise, if copy: pop dst from the head of the free queue (ref 1), drop
 *   one reference of the tail src, replace the tail entry in place, record
 *   (src, dst) as a pending copy that keeps both blocks out of the free queue
 *   until pa_pool_copies_done, and report it in cow_pair_out; then pop
 *   `needed` blocks (ref 1) onto the table, and write the slot of every new
 *   position p in [len, len + n):  slot = table[p / B] * B + p % B.  A block
 *   popped from the free queue loses its cached hash.
 * ("Memory management", Code: append with copy-on-write; "PagedAttention:
 * fragmentation, blocks, block tables": get_new_blocks pops from the head,
 * the block table is append-only, 3. The slot mapping, and the copy-on-write
 * section's in-place redirect with a queued (src, dst) copy.)
 * slots_out: host int64 [n_tokens].  cow_pair_out: host int32 [2], set to
 * {-1, -1} when no copy is needed.  The caller must copy block src to dst
 * (pa_copy_blocks) before any write to dst, then call pa_pool_copies_done
 * once the copies are ordered before later work.
 * Errors: PA_ERR_INVALID (unknown seq, n_tokens < 1, NULL outputs),
 * PA_ERR_NO_SPACE (pool unchanged). */
int pa_pool_append(pa_pool* pool, int64_t seq_id, int32_t n_tokens,
                   int64_t* slots_out, int32_t* cow_pair_out);

/* pa_pool_append for n_seqs sequences in order.  slots_out receives the slots
 * of all sequences concatenated (sum of n_tokens entries); cow_pairs_out is
 * [n_seqs][2].  Stops at the first failing sequence and returns its error;
 * *n_done (required) is the number of sequences appended, whose results stay
 * committed (each single append is all-or-nothing). */
int pa_pool_append_batch(pa_pool* pool, const int64_t* seq_ids, const int32_t* n_tokens,
                         int32_t n_seqs, int64_t* slots_out, int32_t* cow_pairs_out,
                         int32_t* n_done);

/* Release seq_id: walk its blocks from the tail to the head and drop one
 * reference each.  Of the blocks that are left with no reference, no pin and
 * no pending copy, taken in that tail-first order, the unhashed ones go to the
 * head of the free queue (the sequence's tail block is the next one reused)
 * and the hashed ones to its tail (reused last, still matchable by a prefix
 * lookup until popped).
 * ("PagedAttention: fragmentation, blocks, block tables", 1. The block pool:
 * free_blocks receives the blocks in the order they should be reused,
 * puts uncached ones at the front of the queue and cached ones at the back,
 * and a request hands in its blocks tail first.)
 * Errors: PA_ERR_INVALID if seq_id is unknown. */
int pa_pool_free_seq(pa_pool* pool, int64_t seq_id);

/* Pin every block of seq_id for an outgoing transfer transfer_id (a KV
 * transfer to another engine reads them after the sequence may be gone).  A
 * pinned block is not reused while pinned and a partial tail that is pinned is
 * copied before the next write, as a shared one is.  blocks_out (host int32
 * [cap]) receives the pinned ids in table order and *n_out their number.
 * ("PagedAttention: fragmentation, blocks, block tables", CPU reference
 * allocator: owner references and transfer pins both keep a block live.)
 * Errors: PA_ERR_INVALID for an unknown sequence, an existing transfer_id or
 * too small a cap (*n_out says how many are needed; nothing pinned). */
int pa_pool_pin(pa_pool* pool, int64_t seq_id, int64_t transfer_id, int32_t* blocks_out,
                int32_t cap, int32_t* n_out);

/* End transfer transfer_id: drop its pins, releasing (as pa_pool_free_seq
 * does, last pinned block first) the blocks left with no reference, pin or
 * pending copy.  Errors: PA_ERR_INVALID if transfer_id is unknown. */
int pa_pool_unpin(pa_pool* pool, int64_t transfer_id);

/* The copies reported by pa_pool_append since the last call have been issued
 * (on the stream that orders them before later kernels): release every copy's
 * source and destination hold, freeing the blocks left with nothing else
 * retaining them.  (Copy-on-write section: the scheduler issues the queued
 * copies before the step's kernels.) */
int pa_pool_copies_done(pa_pool* pool);

/* Write the block tables of n_seqs sequences into table_out (host int32
 * [n_seqs][bt_stride]): row i gets ceil(len_i / B) block ids; the rest of the
 * row is not written.  seq_lens_out (host int32 [n_seqs], nullable) gets the
 * lengths.  Errors: PA_ERR_INVALID for an unknown sequence, a row longer than
 * bt_stride or a length above INT32_MAX (nothing written). */
int pa_pool_block_table(const pa_pool* pool, const int64_t* seq_ids, int32_t n_seqs,
                        int32_t* table_out, int32_t bt_stride, int32_t* seq_lens_out);

/* pa_pool_block_table for a kernel that wants smaller pages: every
 * allocation block b of a row (block_size tokens) is written as the k =
 * block_size / kernel_block_size kernel blocks b*k .. b*k + k - 1, which are
 * the same memory when the cache is viewed with kernel_block_size-token
 * blocks ([num_blocks * k][kernel_block_size][Hkv][D]).  Row i gets
 * ceil(len_i / block_size) * k entries; slots are unchanged by the view.
 * ("PagedAttention: fragmentation, blocks, block tables", the block-table
 * append with hybrid blocks, and the paragraph on decoupling the allocation
 * block from the kernel block: the allocator's block size and the one an
 * attention kernel is tuned for need not be equal when the first is a
 * multiple of the second.)
 * Errors: PA_ERR_INVALID if kernel_block_size does not divide block_size, a
 * row does not fit bt_stride, num_blocks * k exceeds INT32_MAX or a sequence
 * is unknown (nothing written). */
int pa_pool_kernel_block_table(const pa_pool* pool, const int64_t* seq_ids, int32_t n_seqs,
                               int32_t kernel_block_size, int32_t* table_out, int32_t bt_stride,
                               int32_t* seq_lens_out);

/* Number of free blocks (the capacity test is a subtraction against it). */
int pa_pool_num_free(const pa_pool* pool, int32_t* out);
/* Pool usage, into out[0..4]: blocks in use (owned, pinned or held for a
 * pending copy), free blocks, cached block hashes, tokens over all sequences,
 * and tail waste -- slots of the sequences' blocks not holding a token,
 * sum over sequences of B * ceil(len / B) - len (a block shared by forked
 * sequences counts once per sequence).  ("PagedAttention: fragmentation,
 * blocks, block tables": the waste is bounded by the last block of each
 * sequence; "The pantry of pigeonholes", The maths that matter: waste =
 * B ceil(n / B) - n.)  Errors: PA_ERR_INVALID for a NULL pool or out, or
 * n_out < 5. */
int pa_pool_stats(const pa_pool* pool, int64_t* out, int32_t n_out);
/* Number of cached block hashes (each names one block, free or in use). */
int pa_pool_num_cached(const pa_pool* pool, int32_t* out);
/* Pins, pending copies and cached hash of block_id (*hashed_out 0 or 1; the
 * hash is 0 when not hashed).  Errors: PA_ERR_INVALID if out of range. */
int pa_pool_block_state(const pa_pool* pool, int32_t block_id, int32_t* pins_out,
                        int32_t* pending_out, uint64_t* hash_out, int32_t* hashed_out);
/* Reference count of block_id.  Errors: PA_ERR_INVALID if out of range. */
int pa_pool_refcount(const pa_pool* pool, int32_t block_id, int32_t* out);
/* Token count of seq_id. */
int pa_pool_seq_len(const pa_pool* pool, int64_t seq_id, int64_t* out);
/* The free queue from head to tail: writes min(cap, free) ids, *n_out = free. */
int pa_pool_free_order(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out);

/* Check the allocator invariants (CPU reference allocator section): a block is
 * in the free queue exactly when it has no reference, pin or pending copy, and
 * the queue's links are consistent; every table entry is a valid id whose
 * reference count equals its number of owners; pin and pending-copy counts
 * equal their records; no table repeats a block; each table holds exactly
 * ceil(len / B) blocks; the hash map and the blocks' hashes name each other.
 * Returns PA_OK or PA_ERR_INVALID with the first violation in pa_last_error. */
int pa_pool_check(const pa_pool* pool);

/* Blocks that fit in pool_bytes: floor(floor(pool_bytes / bytes_per_token) /
 * block_size) -- the two floor divisions of the first page's budget
 * paragraph.  Returns -1 for non-positive bytes_per_token or block_size or a
 * negative pool_bytes. */
int64_t pa_blocks_for_bytes(int64_t pool_bytes, int64_t bytes_per_token, int32_t block_size);

/* ------------------------------------------------------------------------ */
/* Device calls (gfx950), asynchronous on `stream`                           */
/* ------------------------------------------------------------------------ */

/* Compute the step's slot mapping on the device from the block table.
 * Request i owns step tokens query_start_loc[i] .. query_start_loc[i+1]-1,
 * the last q_i = query_start_loc[i+1] - query_start_loc[i] of its
 * seq_lens[i] positions: token query_start_loc[i] + j sits at position
 * p = seq_lens[i] - q_i + j and gets
 *   slot_mapping[query_start_loc[i] + j] = block_tables[i][p / B] * B + p % B.
 * Tokens from query_start_loc[num_seqs] up to num_tokens (padding), a
 * negative p and p / B >= bt_stride get the padding id -1.
 * ("PagedAttention: fragmentation, blocks, block tables", 3. The slot mapping:
 * with one context-parallel rank the slot kernel reduces to this formula;
 * attention-metadata section for query_start_loc and seq_lens.)
 * slot_mapping: device int64 [num_tokens] (written).  block_tables: device
 * int32, row i at block_tables + i * bt_stride.  query_start_loc: device int32
 * [num_seqs + 1], non-decreasing, query_start_loc[num_seqs] <= num_tokens is
 * not required (tokens past num_tokens are not written).  seq_lens: device
 * int32 [num_seqs].  block_size: power of two <= 256.
 * Errors: PA_ERR_INVALID for NULL pointers, negative counts, bt_stride < 1 or
 * a bad block_size.  Integer work, bit-exact. */
int pa_slot_mapping(int64_t* slot_mapping, int32_t num_tokens,
                    const int32_t* block_tables, int32_t bt_stride,
                    const int32_t* query_start_loc, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t block_size, void* stream);

/* Store each new token's K and V rows at its slot: row t of key/value
 * ([num_tokens][num_kv_heads][head_dim] bf16, consecutive tokens
 * key_row_stride / value_row_stride elements apart, heads contiguous) goes to
 * slot slot_mapping[t], i.e. block slot / B at offset slot % B.  A slot of -1
 * (the padding id) -- or any slot outside [0, num_blocks * B) -- is skipped.
 * Slots must be unique within a call.
 * ("PagedAttention: fragmentation, blocks, block tables", 3. The slot mapping:
 * one int64 per scheduled token, a flat index into block-major storage, the
 * padding id for tokens without a slot; worked allocation, step 9.)
 * All pointers are device pointers, 16-byte aligned; strides multiples of 8.
 * Bit-exact copy. */
int pa_reshape_and_cache(const void* key, int64_t key_row_stride,
                         const void* value, int64_t value_row_stride,
                         void* key_cache, void* value_cache, int64_t cache_block_stride,
                         int32_t num_blocks, const int64_t* slot_mapping,
                         int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, void* stream);

/* pa_reshape_and_cache into E4M3 caches (one byte per element): each bf16
 * element x is stored as the E4M3 code of the fp32 product x * r, where
 * r = fp32(1 / k_scale) for K and fp32(1 / v_scale) for V; the code's value
 * times the scale stands for x.  E4M3 here is the finite-only form (bias 7,
 * subnormals m * 2^-9, largest finite 448, S.1111.111 = NaN); rounding is to
 * nearest, ties to even; magnitudes above 448 saturate to +-448; NaN stays NaN.
 * ("The pantry of pigeonholes", knobs table and "With KV quantisation": an
 * FP8 KV cache halves the bytes per token.  Format, scaling and rounding are
 * not given there; the ones above are this library's.)
 * key_cache / value_cache: device uint8 [num_blocks][block_size][num_kv_heads]
 * [head_dim] codes, block b at b * cache_block_stride bytes (a multiple of 16).
 * Errors as pa_reshape_and_cache, plus PA_ERR_INVALID for a scale that is not
 * positive and finite. */
int pa_reshape_and_cache_fp8(const void* key, int64_t key_row_stride,
                             const void* value, int64_t value_row_stride,
                             void* key_cache, void* value_cache, int64_t cache_block_stride,
                             int32_t num_blocks, const int64_t* slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float k_scale, float v_scale, void* stream);

/* A decode step's cache write that also keeps device block tables current:
 * row i (i < num_rows) has one new token whose K and V rows are row i of
 * key/value (as in pa_reshape_and_cache), whose slot is slots[i] (the slot
 * pa_pool_append returned for it) and whose position is positions[i] = p
 * (the row's length before the step).  The call writes the token to its
 * slot, sets block_tables[i][p / B] = slots[i] / B and seq_lens[i] = p + 1.
 * By the slot formula that entry is the block the pool put position p in,
 * so the device table follows the host pool -- a newly allocated block, or
 * the in-place redirect of a copied tail -- with no host-to-device copy:
 * slots and positions travel in the kernel arguments.  A slot of -1 leaves
 * row i unchanged; an entry p / B >= bt_stride is not written (size the
 * table for the longest sequence).  Run pa_copy_blocks for the step's pairs
 * first, as for pa_reshape_and_cache.
 * ("PagedAttention: fragmentation, blocks, block tables", 2. The block table
 * (append-only rows), 3. The slot mapping, and the copy-on-write section.)
 * key/value: device bf16 [num_rows][num_kv_heads][head_dim] rows.
 * block_tables: device int32 [num_rows][bt_stride]; seq_lens: device int32
 * [num_rows] (both written); slots: HOST int64 [num_rows]; positions: HOST
 * int32 [num_rows].
 * Errors as pa_reshape_and_cache, plus PA_ERR_INVALID for a negative position
 * of a row with a slot (nothing is launched on an error). */
int pa_decode_append(const void* key, int64_t key_row_stride,
                     const void* value, int64_t value_row_stride,
                     void* key_cache, void* value_cache, int64_t cache_block_stride,
                     int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
                     int32_t* seq_lens, const int64_t* slots, const int32_t* positions,
                     int32_t num_rows, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     void* stream);

/* Copy whole blocks: for every cache c and pair (src, dst),
 * bytes [0, block_bytes) of block dst <- the same bytes of block src, where
 * block b of cache c starts at caches[c] + b * cache_block_stride_bytes.
 * All sources are read before any destination is written.
 * ("PagedAttention: fragmentation, blocks, block tables", copy-on-write
 * section: the pairs travel from the scheduler as (src, dst) ids and one
 * copy covers every byte of the block in every listed tensor.)
 * caches: HOST array of n_caches device pointers.  pairs: HOST int32
 * [n_pairs][2] (src, dst), e.g. the pairs pa_pool_append returned; the library
 * passes them to the kernel by value, so no staging copy is needed.
 * Errors: PA_ERR_INVALID for an id outside [0, num_blocks), a destination
 * named twice, a destination that is also a source, block_bytes not a
 * positive multiple of 16 or above the stride, or unaligned pointers. */
int pa_copy_blocks(void* const* caches, int32_t n_caches, int64_t block_bytes,
                   int64_t cache_block_stride_bytes, int32_t num_blocks,
                   const int32_t* pairs, int32_t n_pairs, void* stream);

/* pa_copy_blocks with the pairs in device memory, for launches captured once
 * and replayed with new pairs (a HIP graph): pairs is a device int32
 * [n_pairs][2] (src, dst) array read by the kernel; a pair with an id outside
 * [0, num_blocks) is skipped, so -1 pads a list to a fixed n_pairs.  The
 * pairs cannot be checked on the host: a destination named twice, or a
 * destination that is also a source, gives an unspecified result (every
 * access still stays inside the listed caches).  Every byte of each block is
 * copied, as by pa_copy_blocks.  Errors: PA_ERR_INVALID for NULL or
 * unaligned pointers and bad sizes (as pa_copy_blocks). */
int pa_copy_blocks_device(void* const* caches, int32_t n_caches, int64_t block_bytes,
                          int64_t cache_block_stride_bytes, int32_t num_blocks,
                          const int32_t* pairs, int32_t n_pairs, void* stream);

/* Bytes of workspace pa_paged_decode needs (0 when one partition covers
 * max_seq_len, i.e. no split). */
size_t pa_paged_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_seq_len,
                                      int32_t partition_size);

/* Single-query attention per sequence over its paged K/V.
 * For sequence s and query head h (KV head g = h / (num_q_heads/num_kv_heads)):
 *   x_t = scale * <q[s,h], K_t>  for the seq_lens[s] tokens t of the sequence,
 *   out[s,h] = sum_t softmax(x)_t V_t   (bf16), lse[s,h] = ln sum_t exp(x_t),
 * where token t is row t % B of block block_tables[s][t / B].
 * ("PagedAttention: fragmentation, blocks, block tables", attention-metadata
 * section: the kernel gathers past K/V by walking row s of the block table for
 * ceil(seq_lens[s] / B) entries; seq_lens counts the tokens already written,
 * including this step's.  Split-K, named there without detail: partition p
 * covers tokens [p*P, (p+1)*P) and partitions are merged with the
 * log-sum-exp identity.)
 * q, out: device bf16 [num_seqs][num_q_heads][head_dim], contiguous.
 * lse: device fp32 [num_seqs][num_q_heads] or NULL.
 * seq_lens: device int32 [num_seqs]; each must be <= max_seq_len.  The
 * lengths live on the device, so the call cannot check them: a longer
 * sequence is attended over its first max_seq_len tokens only (and a
 * negative length counts as 0), which keeps every read inside the table and
 * the cache but is a wrong answer for that row.  A length of 0 yields out = 0
 * and lse = -inf.  ceil(max_seq_len / B) must not exceed bt_stride.
 * partition_size: 0 = one partition per sequence; otherwise a multiple of 64
 * and of block_size.  workspace: device buffer of at least
 * pa_paged_decode_workspace_size(...) bytes (may be NULL when that is 0),
 * 256-byte aligned; its contents on entry do not matter.
 * Arithmetic: fp32 accumulation of bf16 products; softmax weights are rounded
 * to bf16 before they multiply V. */
int pa_paged_decode(void* out, float* lse, const void* q,
                    const void* key_cache, const void* value_cache,
                    int64_t cache_block_stride, int32_t num_blocks,
                    const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                    int32_t partition_size, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* pa_paged_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and result, without the workspace.  The split-K partials
 * go to a scratch array of PA_STATIC_SCRATCH_BYTES (64 MiB) that the library
 * keeps in device memory; every GPU the library runs on holds its own copy
 * until the process ends.  The call itself allocates nothing.  All calls on
 * one GPU share that GPU's scratch: calls that overlap in time on one GPU
 * (different streams, no ordering between them) race; calls ordered on one
 * stream do not.  Nothing carries over between calls (each call writes every
 * partial it reads), so the scratch needs no clearing.
 * Errors as pa_paged_decode, plus PA_ERR_INVALID when the call needs more
 * partials than the scratch holds (pa_paged_decode_workspace_size above
 * PA_STATIC_SCRATCH_BYTES); nothing is launched then. */
#define PA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int pa_paged_decode_noalloc(void* out, float* lse, const void* q,
                            const void* key_cache, const void* value_cache,
                            int64_t cache_block_stride, int32_t num_blocks,
                            const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                            int32_t partition_size, float scale, void* stream);

/* pa_decode_append followed by pa_paged_decode, in one launch per 256
 * sequences: row s's new token (K/V rows = row s of key/value, slot
 * slots[s], position positions[s]) is written to the cache, block_tables[s]
 * [positions[s] / B] becomes slots[s] / B and seq_lens[s] becomes
 * positions[s] + 1, and the row attends over all positions[s] + 1 tokens.
 * Every work-group of a row takes the row's length and the new position's
 * block from the host arrays and reads the new token from key/value, so none
 * reads what the launch writes; rows with slot -1 are plain decode rows
 * (seq_lens[s] as stored).  Run pa_copy_blocks for the step's pairs first.
 * ("PagedAttention: fragmentation, blocks, block tables", 2. The block table,
 * 3. The slot mapping, the copy-on-write section and the attention-metadata
 * section.)
 * Arguments as pa_paged_decode and pa_decode_append (slots, positions: HOST
 * arrays of num_seqs entries; block_tables and seq_lens are written);
 * bf16 caches only.  Errors as those two, plus PA_ERR_INVALID for a
 * position outside [0, max_seq_len) or a slot past the pool. */
int pa_paged_decode_append(void* out, float* lse, const void* q,
                           void* key_cache, void* value_cache,
                           int64_t cache_block_stride, int32_t num_blocks,
                           int32_t* block_tables, int32_t bt_stride, int32_t* seq_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                           int32_t partition_size, float scale,
                           const void* key, int64_t key_row_stride,
                           const void* value, int64_t value_row_stride,
                           const int64_t* slots, const int32_t* positions,
                           void* workspace, size_t workspace_bytes, void* stream);

/* pa_paged_decode over E4M3 caches written by pa_reshape_and_cache_fp8: K_t
 * and V_t above are the codes' values times k_scale and v_scale.  Codes are
 * converted to bf16 exactly; the logits use scale * k_scale (rounded to fp32)
 * and the output is multiplied by v_scale.  cache_block_stride is in bytes
 * and must be a multiple of 16.  Same workspace as pa_paged_decode.
 * ("The pantry of pigeonholes", knobs table and "With KV quantisation".)
 * Errors as pa_paged_decode, plus PA_ERR_INVALID for a scale that is not
 * positive and finite. */
int pa_paged_decode_fp8(void* out, float* lse, const void* q,
                        const void* key_cache, const void* value_cache,
                        int64_t cache_block_stride, int32_t num_blocks,
                        const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                        int32_t partition_size, float scale, float k_scale, float v_scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Chunked-prefill attention of query chunks over their paged context.
 * Request i's queries are rows query_start_loc[i] .. query_start_loc[i+1]-1 of
 * q; they are the last q_i = query_start_loc[i+1] - query_start_loc[i] tokens
 * of its seq_lens[i] tokens, already written to the cache.  Query j of request
 * i (absolute position c_i + j, c_i = seq_lens[i] - q_i) attends to keys
 * 0 .. c_i + j when causal != 0, else to all seq_lens[i] keys.
 * ("PagedAttention: fragmentation, blocks, block tables", attention-metadata
 * section: query_start_loc, seq_lens, max_query_len, max_seq_len, the block
 * table and the gather by table walk.)
 * q, out: device bf16 [total_q][num_q_heads][head_dim], contiguous, with
 * total_q = query_start_loc[num_seqs].  query_start_loc: device int32
 * [num_seqs + 1], non-decreasing, starting at 0; seq_lens: device int32
 * [num_seqs] with q_i <= seq_lens[i] <= max_seq_len; max_query_len bounds
 * every q_i.  ceil(max_seq_len / B) must not exceed bt_stride.  These
 * device arrays cannot be checked by the call; when they break the bounds,
 * no read leaves the table or the cache, but rows go unwritten: the queries
 * of a request past its first max_query_len, and every query of a request
 * with q_i > seq_lens[i] (lengths above max_seq_len are cut to it first).
 * pa_paged_attention, which also takes the host copy of query_start_loc,
 * rejects a q_i above max_query_len.
 * Arithmetic: bf16 MFMA products with fp32 accumulation; softmax weights are
 * rounded to bf16 before the PV product. */
int pa_paged_prefill(void* out, const void* q,
                     const void* key_cache, const void* value_cache,
                     int64_t cache_block_stride, int32_t num_blocks,
                     const int32_t* block_tables, int32_t bt_stride,
                     const int32_t* query_start_loc, const int32_t* seq_lens,
                     int32_t num_seqs, int32_t max_query_len, int32_t max_seq_len,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, float scale, int32_t causal, void* stream);

/* pa_paged_prefill over E4M3 caches written by pa_reshape_and_cache_fp8: K
 * and V are the codes' values times k_scale and v_scale.  Each key tile's
 * codes become bf16 exactly while they are staged; the logits use
 * scale * k_scale (rounded to fp32) and the output is multiplied by v_scale.
 * cache_block_stride is in bytes and must be a multiple of 16.
 * ("The pantry of pigeonholes", knobs table and "With KV quantisation".)
 * Errors as pa_paged_prefill, plus PA_ERR_INVALID for a scale that is not
 * positive and finite. */
int pa_paged_prefill_fp8(void* out, const void* q,
                         const void* key_cache, const void* value_cache,
                         int64_t cache_block_stride, int32_t num_blocks,
                         const int32_t* block_tables, int32_t bt_stride,
                         const int32_t* query_start_loc, const int32_t* seq_lens,
                         int32_t num_seqs, int32_t max_query_len, int32_t max_seq_len,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, float scale, float k_scale, float v_scale,
                         int32_t causal, void* stream);

/* Bytes of workspace pa_paged_attention needs for a batch: that of
 * pa_paged_decode for the batch's decode rows (the leading requests with one
 * query each, found from query_start_loc_host); 0 when none is split. */
size_t pa_paged_attention_workspace_size(const int32_t* query_start_loc_host, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                                         int32_t partition_size);

/* A whole step's attention -- prefill chunks and decode rows of a mixed batch
 * -- in one launch (plus the merge pass of decode rows split into
 * partitions).  One metadata set describes every request, as in the
 * attention-metadata section of "PagedAttention: fragmentation, blocks,
 * block tables": request i's queries are rows query_start_loc[i] ..
 * query_start_loc[i+1]-1 of q, the last q_i of its seq_lens[i] tokens (all
 * written to the cache), and query j attends to keys 0 .. c_i + j (causal,
 * c_i = seq_lens[i] - q_i) or to all seq_lens[i] keys, gathered by walking
 * row i of the block table; a decode is a request with one query.
 * The leading requests with one query each (the decode rows; with the usual
 * decode-first batch order, all of them) run the pa_paged_decode partition
 * pass with partition_size; the others run the pa_paged_prefill body; both
 * kinds' work-groups share one grid, so the HBM-bound decode and the
 * MFMA-bound prefill run side by side.  Results are bit for bit those of
 * pa_paged_decode and pa_paged_prefill on the two parts.  (With head_dim
 * 128 and more than 5 query heads per KV head the two parts are launched one
 * after the other.)
 * q, out: device bf16 [total_q][num_q_heads][head_dim], contiguous.
 * query_start_loc: device int32 [num_seqs + 1]; query_start_loc_host: the
 * same values in host memory (the metadata's CPU copy; the launch splits the
 * batch with it).  seq_lens: device int32 [num_seqs].  Every q_i must be at
 * most max_query_len; seq_lens[i] <= max_seq_len; ceil(max_seq_len / B)
 * must not exceed bt_stride.  workspace: at least
 * pa_paged_attention_workspace_size(...) bytes, 256-byte aligned.
 * bf16 caches only.
 * Errors: PA_ERR_INVALID for a query_start_loc_host that does not start at 0
 * or decreases, a request with more than max_query_len queries, and the
 * errors of pa_paged_decode and pa_paged_prefill; nothing is launched then. */
int pa_paged_attention(void* out, const void* q,
                       const void* key_cache, const void* value_cache,
                       int64_t cache_block_stride, int32_t num_blocks,
                       const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* query_start_loc, const int32_t* query_start_loc_host,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t max_query_len,
                       int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t partition_size, float scale,
                       int32_t causal, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
