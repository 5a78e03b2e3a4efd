// Host block pool: free queue, reference counts, append-only block tables,
// ceil(n/B) allocation, copy-on-write of a shared partial tail, prefix
// caching by block hash, and transfer pins.
//
// "PagedAttention: fragmentation, blocks, block tables":
//   1. The block pool -- every physical block has metadata (id, refcount, the
//      hash of its contents once cached) and sits in one free queue at
//      construction; allocation pops from the head and evicts the popped
//      block's cached hash; freeing drops a reference and, at zero, returns an
//      unhashed block to the front (reused first) and a hashed one to the back
//      (reused last, still matchable), in eviction-priority order, a request
//      freeing its blocks tail first.  The queue is intrusive, so a block that
//      a prefix hit touches leaves the middle of the queue in O(1).
//   2. The block table -- position p is in block table[p / B] at p % B.
//   3. The slot mapping -- slot = table[p / B] * B + p % B.
//   copy-on-write section -- the shared tail entry is replaced in place by a
//      private block and the (src, dst) pair is handed to the caller; both
//      endpoints stay retained until the copy has run (the caller reports it);
//      a full-block prefix hit just touches the block.
//   CPU reference allocator -- owner references and transfer pins: a block is
//      reusable only when it has neither; a pinned partial tail is copied
//      before a write, like a shared one.
// "The pantry of pigeonholes", prefix sharing -- a block's hash covers its
//   tokens and the previous block's hash, so it captures position.
// "Memory management", Code -- append with copy-on-write: the capacity test
//   covers the copy block and the new blocks before anything changes.
// Kernel blocks (the block-table append's hybrid branch and the decoupling
//   paragraph of the first page): an allocation block of B tokens is the
//   same memory as k = B / B_kernel kernel blocks, ids b*k .. b*k + k - 1.
//
// Readings: the hash is 64-bit FNV-1a over the parent hash (8 bytes LE, 0 for
// the first block) and the block's token ids (4 bytes LE each); only full
// blocks are hashed and matched; the first block entered for a hash keeps it.
#include <algorithm>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "internal.hpp"
#include "pagedattn.h"

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // intrusive doubly linked free queue over block ids (-1 = none)
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> queued;
  int32_t head = -1, tail = -1, count = 0;
  std::vector<int32_t> ref;   // owners: tables naming the block
  std::vector<int32_t> pins;  // transfer pins
  std::vector<int32_t> hold;  // pending copy-on-write copies
  std::vector<uint8_t> hashed;
  std::vector<uint64_t> hash;
  std::unordered_map<uint64_t, int32_t> cached;                  // hash -> block
  std::unordered_map<int64_t, std::vector<int32_t>> transfers;   // id -> pinned blocks
  std::vector<std::pair<int32_t, int32_t>> pending;              // copies not yet run
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  bool retained(int32_t b) const { return ref[(size_t)b] + pins[(size_t)b] + hold[(size_t)b] > 0; }

  void push_front(int32_t b) {
    prev[(size_t)b] = -1;
    next[(size_t)b] = head;
    if (head >= 0) prev[(size_t)head] = b; else tail = b;
    head = b;
    queued[(size_t)b] = 1;
    ++count;
  }
  void push_back(int32_t b) {
    next[(size_t)b] = -1;
    prev[(size_t)b] = tail;
    if (tail >= 0) next[(size_t)tail] = b; else head = b;
    tail = b;
    queued[(size_t)b] = 1;
    ++count;
  }
  void remove(int32_t b) {  // O(1) removal from anywhere in the queue
    const int32_t p = prev[(size_t)b], n = next[(size_t)b];
    if (p >= 0) next[(size_t)p] = n; else head = n;
    if (n >= 0) prev[(size_t)n] = p; else tail = p;
    queued[(size_t)b] = 0;
    --count;
  }
  // Head of the queue, its cached hash (if any) evicted.
  int32_t pop() {
    const int32_t b = head;
    remove(b);
    if (hashed[(size_t)b]) {
      cached.erase(hash[(size_t)b]);
      hashed[(size_t)b] = 0;
    }
    return b;
  }
  // A block gains an owner; a free (evictable) block leaves the queue.
  void touch(int32_t b) {
    if (!retained(b)) remove(b);
    ref[(size_t)b] += 1;
  }
  // `blocks` (eviction-priority order) have just lost their last reference:
  // unhashed ones to the head, hashed ones to the tail, each group in order.
  void release(const std::vector<int32_t>& blocks) {
    for (auto it = blocks.rbegin(); it != blocks.rend(); ++it)
      if (!hashed[(size_t)*it]) push_front(*it);
    for (int32_t b : blocks)
      if (hashed[(size_t)b]) push_back(b);
  }
};

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 64-bit FNV-1a over the parent hash (8 bytes, little-endian) and the block's
// token ids (4 bytes each, little-endian, two's complement).
constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

uint64_t block_hash(uint64_t parent, const int32_t* tokens, int32_t n) {
  uint64_t h = kFnvOffset;
  for (int i = 0; i < 8; ++i) {
    h ^= (parent >> (8 * i)) & 0xff;
    h *= kFnvPrime;
  }
  for (int32_t t = 0; t < n; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xff;
      h *= kFnvPrime;
    }
  }
  return h;
}

// All-or-nothing append of one sequence.  Host memory for the table and the
// pending-copy record grows before any pool state changes, so an allocation
// failure leaves it intact.
int append_one(pa_pool* p, int64_t seq_id, int32_t n, int64_t* slots, int32_t* pair) {
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return pa::fail(PA_ERR_INVALID, "append: unknown sequence %lld", (long long)seq_id);
  if (n < 1) return pa::fail(PA_ERR_INVALID, "append: n_tokens must be >= 1 (got %d)", n);
  pa_pool::Seq& s = it->second;
  const int64_t B = p->block_size;
  const int64_t L = s.len;
  if (L > INT64_MAX - n) return pa::fail(PA_ERR_INVALID, "append: length overflow");
  const int64_t needed = cdiv(L + n, B) - (int64_t)s.blocks.size();
  const int32_t last = s.blocks.empty() ? -1 : s.blocks.back();
  const bool cow = (L % B != 0) && (p->ref[(size_t)last] > 1 || p->pins[(size_t)last] > 0);
  if (needed + (cow ? 1 : 0) > p->count)
    return pa::fail(PA_ERR_NO_SPACE, "append: need %lld blocks, %d free",
                    (long long)(needed + (cow ? 1 : 0)), p->count);
  try {
    s.blocks.reserve(s.blocks.size() + (size_t)needed);
    if (cow) p->pending.reserve(p->pending.size() + 1);
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "append: out of host memory");
  }
  pair[0] = -1;
  pair[1] = -1;
  if (cow) {
    const int32_t src = last;
    const int32_t dst = p->pop();
    p->ref[(size_t)dst] = 1;
    p->ref[(size_t)src] -= 1;
    p->hold[(size_t)src] += 1;
    p->hold[(size_t)dst] += 1;
    p->pending.emplace_back(src, dst);
    s.blocks.back() = dst;
    pair[0] = src;
    pair[1] = dst;
  }
  for (int64_t i = 0; i < needed; ++i) {
    const int32_t b = p->pop();
    p->ref[(size_t)b] = 1;
    s.blocks.push_back(b);
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t pos = L + i;
    slots[i] = (int64_t)s.blocks[(size_t)(pos / B)] * B + pos % B;
  }
  s.len = L + n;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* order, pa_pool** out) {
  pa::clear_error();
  if (!out) return pa::fail(PA_ERR_INVALID, "pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_INVALID, "pool_create: num_blocks (%d) and block_size (%d) must be positive",
                    num_blocks, block_size);
  pa_pool* p = new (std::nothrow) pa_pool();
  if (!p) return pa::fail(PA_ERR_NO_MEMORY, "pool_create: out of host memory");
  const size_t N = (size_t)num_blocks;
  try {
    p->prev.assign(N, -1);
    p->next.assign(N, -1);
    p->queued.assign(N, 0);
    p->ref.assign(N, 0);
    p->pins.assign(N, 0);
    p->hold.assign(N, 0);
    p->hashed.assign(N, 0);
    p->hash.assign(N, 0);
  } catch (const std::bad_alloc&) {
    delete p;
    return pa::fail(PA_ERR_NO_MEMORY, "pool_create: out of host memory");
  }
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  if (order) {
    std::vector<char> seen(N, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
        delete p;
        return pa::fail(PA_ERR_INVALID, "pool_create: initial order is not a permutation (entry %d = %d)", i, b);
      }
      seen[(size_t)b] = 1;
    }
    for (int32_t i = 0; i < num_blocks; ++i) p->push_back(order[i]);
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->push_back(i);
  }
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

int pa_pool_add_seq(pa_pool* p, int64_t seq_id) {
  pa::clear_error();
  if (!p) return pa::fail(PA_ERR_INVALID, "add_seq: pool is NULL");
  if (p->seqs.count(seq_id)) return pa::fail(PA_ERR_INVALID, "add_seq: sequence %lld exists", (long long)seq_id);
  try {
    p->seqs.emplace(seq_id, pa_pool::Seq());
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "add_seq: out of host memory");
  }
  return PA_OK;
}

int pa_pool_add_seq_cached(pa_pool* p, int64_t seq_id, const int32_t* tokens, int64_t n_tokens,
                           int64_t* hit_tokens) {
  pa::clear_error();
  if (!p || !hit_tokens || n_tokens < 0 || (n_tokens > 0 && !tokens))
    return pa::fail(PA_ERR_INVALID, "add_seq_cached: bad argument");
  *hit_tokens = 0;
  if (p->seqs.count(seq_id))
    return pa::fail(PA_ERR_INVALID, "add_seq_cached: sequence %lld exists", (long long)seq_id);
  const int64_t B = p->block_size;
  // the hit blocks first (nothing changes yet), then one insertion
  std::vector<int32_t> hits;
  try {
    uint64_t h = 0;
    for (int64_t j = 0; (j + 1) * B <= n_tokens; ++j) {
      h = block_hash(h, tokens + j * B, (int32_t)B);
      auto it = p->cached.find(h);
      if (it == p->cached.end()) break;
      hits.push_back(it->second);
    }
    pa_pool::Seq s;
    s.blocks = hits;
    s.len = (int64_t)hits.size() * B;
    p->seqs.emplace(seq_id, std::move(s));
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "add_seq_cached: out of host memory");
  }
  for (int32_t b : hits) p->touch(b);
  *hit_tokens = (int64_t)hits.size() * B;
  return PA_OK;
}

int pa_pool_cache_blocks(pa_pool* p, int64_t seq_id, const int32_t* tokens, int64_t n_tokens) {
  pa::clear_error();
  if (!p || n_tokens < 0 || (n_tokens > 0 && !tokens)) return pa::fail(PA_ERR_INVALID, "cache_blocks: bad argument");
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end())
    return pa::fail(PA_ERR_INVALID, "cache_blocks: unknown sequence %lld", (long long)seq_id);
  const pa_pool::Seq& s = it->second;
  if (n_tokens > s.len)
    return pa::fail(PA_ERR_INVALID, "cache_blocks: %lld tokens but the sequence holds %lld", (long long)n_tokens,
                    (long long)s.len);
  const int64_t B = p->block_size;
  std::vector<std::pair<int32_t, uint64_t>> chain;
  try {
    chain.reserve((size_t)(n_tokens / B));
    p->cached.reserve(p->cached.size() + (size_t)(n_tokens / B));
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "cache_blocks: out of host memory");
  }
  uint64_t h = 0;
  for (int64_t j = 0; (j + 1) * B <= n_tokens; ++j) {
    h = block_hash(h, tokens + j * B, (int32_t)B);
    const int32_t b = s.blocks[(size_t)j];
    if (p->hashed[(size_t)b] && p->hash[(size_t)b] != h)
      return pa::fail(PA_ERR_INVALID, "cache_blocks: block %d already holds other content", b);
    chain.emplace_back(b, h);
  }
  for (const auto& bh : chain) {  // all checked: nothing changed on error
    const int32_t b = bh.first;
    if (!p->hashed[(size_t)b] && !p->cached.count(bh.second)) {
      p->cached.emplace(bh.second, b);
      p->hashed[(size_t)b] = 1;
      p->hash[(size_t)b] = bh.second;
    }
  }
  return PA_OK;
}

int pa_pool_fork(pa_pool* p, int64_t src_seq, int64_t dst_seq) {
  pa::clear_error();
  if (!p) return pa::fail(PA_ERR_INVALID, "fork: pool is NULL");
  auto it = p->seqs.find(src_seq);
  if (it == p->seqs.end()) return pa::fail(PA_ERR_INVALID, "fork: unknown sequence %lld", (long long)src_seq);
  if (p->seqs.count(dst_seq)) return pa::fail(PA_ERR_INVALID, "fork: sequence %lld exists", (long long)dst_seq);
  try {
    pa_pool::Seq copy = it->second;
    p->seqs.emplace(dst_seq, std::move(copy));
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "fork: out of host memory");
  }
  for (int32_t b : p->seqs[dst_seq].blocks) p->ref[(size_t)b] += 1;
  return PA_OK;
}

int pa_pool_append(pa_pool* p, int64_t seq_id, int32_t n_tokens, int64_t* slots_out, int32_t* cow_pair_out) {
  pa::clear_error();
  if (!p || !slots_out || !cow_pair_out) return pa::fail(PA_ERR_INVALID, "append: NULL argument");
  return append_one(p, seq_id, n_tokens, slots_out, cow_pair_out);
}

int pa_pool_append_batch(pa_pool* p, const int64_t* seq_ids, const int32_t* n_tokens, int32_t n_seqs,
                         int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_done) {
  pa::clear_error();
  if (!n_done) return pa::fail(PA_ERR_INVALID, "append_batch: n_done is NULL");
  *n_done = 0;
  if (!p || n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !n_tokens || !slots_out || !cow_pairs_out)))
    return pa::fail(PA_ERR_INVALID, "append_batch: bad argument");
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    int rc = append_one(p, seq_ids[i], n_tokens[i], slots_out + off, cow_pairs_out + 2 * (int64_t)i);
    if (rc != PA_OK) return rc;
    off += n_tokens[i];
    *n_done = i + 1;
  }
  return PA_OK;
}

int pa_pool_free_seq(pa_pool* p, int64_t seq_id) {
  pa::clear_error();
  if (!p) return pa::fail(PA_ERR_INVALID, "free_seq: pool is NULL");
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return pa::fail(PA_ERR_INVALID, "free_seq: unknown sequence %lld", (long long)seq_id);
  const std::vector<int32_t>& blocks = it->second.blocks;
  std::vector<int32_t> released;  // blocks losing their last reference, tail first
  try {
    released.reserve(blocks.size());
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "free_seq: out of host memory");
  }
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) {
    p->ref[(size_t)*b] -= 1;
    if (!p->retained(*b)) released.push_back(*b);
  }
  p->release(released);
  p->seqs.erase(it);
  return PA_OK;
}

int pa_pool_pin(pa_pool* p, int64_t seq_id, int64_t transfer_id, int32_t* blocks_out, int32_t cap, int32_t* n_out) {
  pa::clear_error();
  if (!p || !n_out || cap < 0 || (cap > 0 && !blocks_out)) return pa::fail(PA_ERR_INVALID, "pin: bad argument");
  *n_out = 0;
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return pa::fail(PA_ERR_INVALID, "pin: unknown sequence %lld", (long long)seq_id);
  if (p->transfers.count(transfer_id))
    return pa::fail(PA_ERR_INVALID, "pin: transfer %lld exists", (long long)transfer_id);
  const std::vector<int32_t>& blocks = it->second.blocks;
  *n_out = (int32_t)blocks.size();
  if ((int64_t)blocks.size() > cap)
    return pa::fail(PA_ERR_INVALID, "pin: %zu blocks but room for %d", blocks.size(), cap);
  try {
    p->transfers.emplace(transfer_id, blocks);
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "pin: out of host memory");
  }
  for (size_t i = 0; i < blocks.size(); ++i) {
    p->pins[(size_t)blocks[i]] += 1;
    blocks_out[i] = blocks[i];
  }
  return PA_OK;
}

int pa_pool_unpin(pa_pool* p, int64_t transfer_id) {
  pa::clear_error();
  if (!p) return pa::fail(PA_ERR_INVALID, "unpin: pool is NULL");
  auto it = p->transfers.find(transfer_id);
  if (it == p->transfers.end())
    return pa::fail(PA_ERR_INVALID, "unpin: unknown transfer %lld", (long long)transfer_id);
  std::vector<int32_t> released;
  try {
    released.reserve(it->second.size());
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "unpin: out of host memory");
  }
  for (auto b = it->second.rbegin(); b != it->second.rend(); ++b) {
    p->pins[(size_t)*b] -= 1;
    if (!p->retained(*b)) released.push_back(*b);
  }
  p->release(released);
  p->transfers.erase(it);
  return PA_OK;
}

int pa_pool_copies_done(pa_pool* p) {
  pa::clear_error();
  if (!p) return pa::fail(PA_ERR_INVALID, "copies_done: pool is NULL");
  std::vector<int32_t> released;
  try {
    released.reserve(2 * p->pending.size());
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_NO_MEMORY, "copies_done: out of host memory");
  }
  for (const auto& sd : p->pending)
    for (int32_t b : {sd.first, sd.second}) {
      p->hold[(size_t)b] -= 1;
      if (!p->retained(b)) released.push_back(b);
    }
  p->pending.clear();
  p->release(released);
  return PA_OK;
}

int pa_pool_block_table(const pa_pool* p, const int64_t* seq_ids, int32_t n_seqs, int32_t* table_out,
                        int32_t bt_stride, int32_t* seq_lens_out) {
  pa::clear_error();
  if (!p || n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !table_out)) || bt_stride < 0)
    return pa::fail(PA_ERR_INVALID, "block_table: bad argument");
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = p->seqs.find(seq_ids[i]);
    if (it == p->seqs.end())
      return pa::fail(PA_ERR_INVALID, "block_table: unknown sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.blocks.size() > bt_stride)
      return pa::fail(PA_ERR_INVALID, "block_table: sequence %lld holds %zu blocks > bt_stride %d",
                      (long long)seq_ids[i], it->second.blocks.size(), bt_stride);
    if (it->second.len > INT32_MAX)
      return pa::fail(PA_ERR_INVALID, "block_table: sequence length exceeds int32");
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pa_pool::Seq& s = p->seqs.find(seq_ids[i])->second;
    std::copy(s.blocks.begin(), s.blocks.end(), table_out + (int64_t)i * bt_stride);
    if (seq_lens_out) seq_lens_out[i] = (int32_t)s.len;
  }
  return PA_OK;
}

int pa_pool_kernel_block_table(const pa_pool* p, const int64_t* seq_ids, int32_t n_seqs, int32_t kernel_block_size,
                               int32_t* table_out, int32_t bt_stride, int32_t* seq_lens_out) {
  pa::clear_error();
  if (!p || n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !table_out)) || bt_stride < 0)
    return pa::fail(PA_ERR_INVALID, "kernel_block_table: bad argument");
  if (kernel_block_size <= 0 || p->block_size % kernel_block_size != 0)
    return pa::fail(PA_ERR_INVALID, "kernel_block_table: kernel_block_size %d does not divide block_size %d",
                    kernel_block_size, p->block_size);
  const int64_t k = p->block_size / kernel_block_size;
  if ((int64_t)p->num_blocks * k > INT32_MAX)
    return pa::fail(PA_ERR_INVALID, "kernel_block_table: kernel block ids exceed int32");
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = p->seqs.find(seq_ids[i]);
    if (it == p->seqs.end())
      return pa::fail(PA_ERR_INVALID, "kernel_block_table: unknown sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.blocks.size() * k > bt_stride)
      return pa::fail(PA_ERR_INVALID, "kernel_block_table: sequence %lld needs %lld entries > bt_stride %d",
                      (long long)seq_ids[i], (long long)(it->second.blocks.size() * k), bt_stride);
    if (it->second.len > INT32_MAX)
      return pa::fail(PA_ERR_INVALID, "kernel_block_table: sequence length exceeds int32");
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pa_pool::Seq& s = p->seqs.find(seq_ids[i])->second;
    int32_t* row = table_out + (int64_t)i * bt_stride;
    for (size_t j = 0; j < s.blocks.size(); ++j)
      for (int64_t u = 0; u < k; ++u) row[(int64_t)j * k + u] = (int32_t)(s.blocks[j] * k + u);
    if (seq_lens_out) seq_lens_out[i] = (int32_t)s.len;
  }
  return PA_OK;
}

int pa_pool_num_free(const pa_pool* p, int32_t* out) {
  pa::clear_error();
  if (!p || !out) return pa::fail(PA_ERR_INVALID, "num_free: NULL argument");
  *out = p->count;
  return PA_OK;
}

int pa_pool_stats(const pa_pool* p, int64_t* out, int32_t n_out) {
  pa::clear_error();
  if (!p || !out || n_out < 5) return pa::fail(PA_ERR_INVALID, "stats: need a pool and room for 5 values");
  int64_t tokens = 0, held = 0;
  for (const auto& kv : p->seqs) {
    tokens += kv.second.len;
    held += (int64_t)kv.second.blocks.size();
  }
  out[0] = (int64_t)p->num_blocks - p->count;           // blocks in use (owned, pinned or held)
  out[1] = p->count;                                     // free blocks
  out[2] = (int64_t)p->cached.size();                    // cached block hashes
  out[3] = tokens;                                       // tokens over all sequences
  out[4] = held * p->block_size - tokens;                // slots allocated but not yet written
  return PA_OK;
}

int pa_pool_num_cached(const pa_pool* p, int32_t* out) {
  pa::clear_error();
  if (!p || !out) return pa::fail(PA_ERR_INVALID, "num_cached: NULL argument");
  *out = (int32_t)p->cached.size();
  return PA_OK;
}

int pa_pool_refcount(const pa_pool* p, int32_t block_id, int32_t* out) {
  pa::clear_error();
  if (!p || !out) return pa::fail(PA_ERR_INVALID, "refcount: NULL argument");
  if (block_id < 0 || block_id >= p->num_blocks)
    return pa::fail(PA_ERR_INVALID, "refcount: block %d out of range", block_id);
  *out = p->ref[(size_t)block_id];
  return PA_OK;
}

int pa_pool_block_state(const pa_pool* p, int32_t block_id, int32_t* pins_out, int32_t* pending_out,
                        uint64_t* hash_out, int32_t* hashed_out) {
  pa::clear_error();
  if (!p || !pins_out || !pending_out || !hash_out || !hashed_out)
    return pa::fail(PA_ERR_INVALID, "block_state: NULL argument");
  if (block_id < 0 || block_id >= p->num_blocks)
    return pa::fail(PA_ERR_INVALID, "block_state: block %d out of range", block_id);
  *pins_out = p->pins[(size_t)block_id];
  *pending_out = p->hold[(size_t)block_id];
  *hashed_out = p->hashed[(size_t)block_id];
  *hash_out = p->hashed[(size_t)block_id] ? p->hash[(size_t)block_id] : 0;
  return PA_OK;
}

int pa_pool_seq_len(const pa_pool* p, int64_t seq_id, int64_t* out) {
  pa::clear_error();
  if (!p || !out) return pa::fail(PA_ERR_INVALID, "seq_len: NULL argument");
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return pa::fail(PA_ERR_INVALID, "seq_len: unknown sequence %lld", (long long)seq_id);
  *out = it->second.len;
  return PA_OK;
}

int pa_pool_free_order(const pa_pool* p, int32_t* out, int32_t cap, int32_t* n_out) {
  pa::clear_error();
  if (!p || !n_out || cap < 0 || (cap > 0 && !out)) return pa::fail(PA_ERR_INVALID, "free_order: bad argument");
  int32_t i = 0;
  for (int32_t b = p->head; b >= 0 && i < cap; b = p->next[(size_t)b]) out[i++] = b;
  *n_out = p->count;
  return PA_OK;
}

int pa_pool_check(const pa_pool* p) {
  pa::clear_error();
  if (!p) return pa::fail(PA_ERR_INVALID, "check: pool is NULL");
  const int32_t N = p->num_blocks;
  const int64_t B = p->block_size;
  if (p->count < 0 || p->count > N) return pa::fail(PA_ERR_INVALID, "check: free count %d", p->count);
  std::vector<int32_t> owners((size_t)N, 0), pins((size_t)N, 0), hold((size_t)N, 0);
  std::vector<char> in_free((size_t)N, 0);
  int32_t walked = 0, last = -1;
  for (int32_t b = p->head; b >= 0; b = p->next[(size_t)b]) {
    if (b >= N) return pa::fail(PA_ERR_INVALID, "check: free queue holds id %d", b);
    if (in_free[(size_t)b]) return pa::fail(PA_ERR_INVALID, "check: block %d queued twice", b);
    if (p->prev[(size_t)b] != last) return pa::fail(PA_ERR_INVALID, "check: queue links broken at block %d", b);
    in_free[(size_t)b] = 1;
    last = b;
    if (++walked > N) return pa::fail(PA_ERR_INVALID, "check: free queue has a cycle");
  }
  if (walked != p->count || last != p->tail) return pa::fail(PA_ERR_INVALID, "check: free queue count or tail");
  std::vector<char> mark((size_t)N, 0);
  for (const auto& kv : p->seqs) {
    const auto& s = kv.second;
    if ((int64_t)s.blocks.size() != cdiv(s.len, B))
      return pa::fail(PA_ERR_INVALID, "check: sequence %lld has %zu blocks for %lld tokens",
                      (long long)kv.first, s.blocks.size(), (long long)s.len);
    for (int32_t b : s.blocks) {
      if (b < 0 || b >= N) return pa::fail(PA_ERR_INVALID, "check: sequence %lld names block %d", (long long)kv.first, b);
      if (mark[(size_t)b]) return pa::fail(PA_ERR_INVALID, "check: sequence %lld repeats block %d", (long long)kv.first, b);
      mark[(size_t)b] = 1;
      owners[(size_t)b] += 1;
    }
    for (int32_t b : s.blocks) mark[(size_t)b] = 0;
  }
  for (const auto& kv : p->transfers)
    for (int32_t b : kv.second) pins[(size_t)b] += 1;
  for (const auto& sd : p->pending) {
    hold[(size_t)sd.first] += 1;
    hold[(size_t)sd.second] += 1;
  }
  int32_t retained = 0, hashed = 0;
  for (int32_t b = 0; b < N; ++b) {
    if (owners[(size_t)b] != p->ref[(size_t)b])
      return pa::fail(PA_ERR_INVALID, "check: block %d has %d owners but refcount %d", b, owners[(size_t)b],
                      p->ref[(size_t)b]);
    if (pins[(size_t)b] != p->pins[(size_t)b] || hold[(size_t)b] != p->hold[(size_t)b])
      return pa::fail(PA_ERR_INVALID, "check: block %d pin or copy counts do not match their records", b);
    const bool r = p->retained(b);
    if ((bool)in_free[(size_t)b] == r || (bool)p->queued[(size_t)b] != (bool)in_free[(size_t)b])
      return pa::fail(PA_ERR_INVALID, "check: block %d free=%d retained=%d", b, (int)in_free[(size_t)b], (int)r);
    retained += r;
    if (p->hashed[(size_t)b]) {
      ++hashed;
      auto it = p->cached.find(p->hash[(size_t)b]);
      if (it == p->cached.end() || it->second != b)
        return pa::fail(PA_ERR_INVALID, "check: block %d holds a hash the map does not point back to", b);
    }
  }
  if (retained + p->count != N) return pa::fail(PA_ERR_INVALID, "check: free and retained do not cover the pool");
  if (hashed != (int32_t)p->cached.size()) return pa::fail(PA_ERR_INVALID, "check: hash map size %zu, %d hashed blocks",
                                                          p->cached.size(), hashed);
  return PA_OK;
}

int64_t pa_blocks_for_bytes(int64_t pool_bytes, int64_t bytes_per_token, int32_t block_size) {
  if (pool_bytes < 0 || bytes_per_token <= 0 || block_size <= 0) return -1;
  return (pool_bytes / bytes_per_token) / block_size;
}

}  // extern "C"
