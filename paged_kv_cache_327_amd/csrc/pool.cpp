// Host block pool: free queue, reference counts, append-only block tables,
// ceil(n/B) allocation and copy-on-write of a shared partial tail.
//
// "PagedAttention: fragmentation, blocks, block tables":
//   1. The block pool -- every physical block has metadata (id, refcount) and
//      sits in one free queue at construction; allocation pops from the head;
//      freeing drops a reference and returns non-cached blocks to the front,
//      ordered by eviction priority (first evicted first), a request freeing its
//      blocks tail first.
//   2. The block table -- position p is in block table[p / B] at p % B.
//   3. The slot mapping -- slot = table[p / B] * B + p % B.
//   copy-on-write section -- the shared tail entry is replaced in place by a
//      private block and the (src, dst) pair is handed to the caller.
// "Memory management", Code -- append with copy-on-write: the capacity test
//   covers the copy block and the new blocks before anything changes.
//
// The free queue is a ring buffer of capacity num_blocks: a block is queued at
// most once, so it never overflows, and both ends are O(1).
#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "internal.hpp"
#include "pagedattn.h"

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // free queue storage
  int32_t head = 0;           // index of the queue head in `ring`
  int32_t count = 0;          // number of free blocks
  std::vector<int32_t> ref;   // reference count per block
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t pop_front() {
    int32_t b = ring[head];
    head = head + 1 == num_blocks ? 0 : head + 1;
    --count;
    return b;
  }
  void push_front(int32_t b) {
    head = head == 0 ? num_blocks - 1 : head - 1;
    ring[head] = b;
    ++count;
  }
  int32_t at(int32_t i) const {  // i-th block from the head
    int64_t j = (int64_t)head + i;
    if (j >= num_blocks) j -= num_blocks;
    return ring[(size_t)j];
  }
};

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// All-or-nothing append of one sequence.  Host memory for the table grows
// before any pool state changes, so an allocation failure leaves it intact.
int append_one(pa_pool* p, int64_t seq_id, int32_t n, int64_t* slots, int32_t* pair) {
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return pa::fail(PA_ERR_INVALID, "append: unknown sequence %lld", (long long)seq_id);
  if (n < 1) return pa::fail(PA_ERR_INVALID, "append: n_tokens must be >= 1 (got %d)", n);
  pa_pool::Seq& s = it->second;
  const int64_t B = p->block_size;
  const int64_t L = s.len;
  if (L > INT64_MAX - n) return pa::fail(PA_ERR_INVALID, "append: length overflow");
  const int64_t needed = cdiv(L + n, B) - (int64_t)s.blocks.size();
  const bool cow = (L % B != 0) && p->ref[(size_t)s.blocks.back()] > 1;
  if (needed + (cow ? 1 : 0) > p->count)
    return pa::fail(PA_ERR_NO_SPACE, "append: need %lld blocks, %d free",
                    (long long)(needed + (cow ? 1 : 0)), p->count);
  try {
    s.blocks.reserve(s.blocks.size() + (size_t)needed);
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_INVALID, "append: out of host memory");
  }
  pair[0] = -1;
  pair[1] = -1;
  if (cow) {
    const int32_t src = s.blocks.back();
    const int32_t dst = p->pop_front();
    p->ref[(size_t)dst] = 1;
    p->ref[(size_t)src] -= 1;
    s.blocks.back() = dst;
    pair[0] = src;
    pair[1] = dst;
  }
  for (int64_t i = 0; i < needed; ++i) {
    const int32_t b = p->pop_front();
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
  if (!p) return pa::fail(PA_ERR_INVALID, "pool_create: out of host memory");
  try {
    p->ring.resize((size_t)num_blocks);
    p->ref.assign((size_t)num_blocks, 0);
  } catch (const std::bad_alloc&) {
    delete p;
    return pa::fail(PA_ERR_INVALID, "pool_create: out of host memory");
  }
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  if (order) {
    std::vector<char> seen((size_t)num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
        delete p;
        return pa::fail(PA_ERR_INVALID, "pool_create: initial order is not a permutation (entry %d = %d)", i, b);
      }
      seen[(size_t)b] = 1;
      p->ring[(size_t)i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->ring[(size_t)i] = i;
  }
  p->head = 0;
  p->count = num_blocks;
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
    return pa::fail(PA_ERR_INVALID, "add_seq: out of host memory");
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
    return pa::fail(PA_ERR_INVALID, "fork: out of host memory");
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
  // Blocks reaching zero, in release order (tail first).  Pushing them to the
  // front in reverse leaves the first released block at the head.
  std::vector<int32_t> released;
  try {
    released.reserve(blocks.size());
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_INVALID, "free_seq: out of host memory");
  }
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b)
    if (--p->ref[(size_t)*b] == 0) released.push_back(*b);
  for (auto b = released.rbegin(); b != released.rend(); ++b) p->push_front(*b);
  p->seqs.erase(it);
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

int pa_pool_num_free(const pa_pool* p, int32_t* out) {
  pa::clear_error();
  if (!p || !out) return pa::fail(PA_ERR_INVALID, "num_free: NULL argument");
  *out = p->count;
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
  const int32_t n = std::min(cap, p->count);
  for (int32_t i = 0; i < n; ++i) out[i] = p->at(i);
  *n_out = p->count;
  return PA_OK;
}

int pa_pool_check(const pa_pool* p) {
  pa::clear_error();
  if (!p) return pa::fail(PA_ERR_INVALID, "check: pool is NULL");
  const int32_t N = p->num_blocks;
  const int64_t B = p->block_size;
  if (p->count < 0 || p->count > N) return pa::fail(PA_ERR_INVALID, "check: free count %d", p->count);
  std::vector<int32_t> owners((size_t)N, 0);
  std::vector<char> in_free((size_t)N, 0);
  for (int32_t i = 0; i < p->count; ++i) {
    const int32_t b = p->at(i);
    if (b < 0 || b >= N) return pa::fail(PA_ERR_INVALID, "check: free queue holds id %d", b);
    if (in_free[(size_t)b]) return pa::fail(PA_ERR_INVALID, "check: block %d queued twice", b);
    in_free[(size_t)b] = 1;
  }
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
  int32_t allocated = 0;
  for (int32_t b = 0; b < N; ++b) {
    if (owners[(size_t)b] != p->ref[(size_t)b])
      return pa::fail(PA_ERR_INVALID, "check: block %d has %d owners but refcount %d", b, owners[(size_t)b],
                      p->ref[(size_t)b]);
    if ((bool)in_free[(size_t)b] == (p->ref[(size_t)b] > 0))
      return pa::fail(PA_ERR_INVALID, "check: block %d free=%d refcount %d", b, (int)in_free[(size_t)b],
                      p->ref[(size_t)b]);
    if (p->ref[(size_t)b] > 0) ++allocated;
  }
  if (allocated + p->count != N) return pa::fail(PA_ERR_INVALID, "check: free and allocated do not cover the pool");
  return PA_OK;
}

int64_t pa_blocks_for_bytes(int64_t pool_bytes, int64_t bytes_per_token, int32_t block_size) {
  if (pool_bytes < 0 || bytes_per_token <= 0 || block_size <= 0) return -1;
  return (pool_bytes / bytes_per_token) / block_size;
}

}  // extern "C"
