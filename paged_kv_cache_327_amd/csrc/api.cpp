// C-ABI entry points of the device calls: every argument is validated on the
// host before anything is enqueued, then the HIP launcher runs.  Pool entry
// points live in pool.cpp.
#include <cstdarg>
#include <cstdio>
#include <string>
#include <algorithm>
#include <vector>

#include "internal.hpp"
#include "pagedattn.h"

namespace pa {
namespace {
thread_local std::string g_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

void clear_error() { g_error.clear(); }

}  // namespace pa

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) {
  int r = 0;
  while ((int64_t{1} << r) < x) ++r;
  return r;
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_heads(const char* fn, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
  if (head_dim != 64 && head_dim != 128) return pa::fail(PA_ERR_INVALID, "%s: head_dim %d not in {64, 128}", fn, head_dim);
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 8)
    return pa::fail(PA_ERR_INVALID, "%s: num_q_heads %d must be a multiple (<= 8x) of num_kv_heads %d", fn,
                    num_q_heads, num_kv_heads);
  if (!is_pow2(block_size) || block_size > 256)
    return pa::fail(PA_ERR_INVALID, "%s: block_size %d is not a power of two in [1, 256]", fn, block_size);
  return PA_OK;
}

int check_cache(const char* fn, const void* kc, const void* vc, int64_t block_stride, int32_t num_blocks,
                int32_t block_size, int64_t row_elems) {
  if (!kc || !vc) return pa::fail(PA_ERR_INVALID, "%s: NULL cache pointer", fn);
  if (!aligned(kc, 16) || !aligned(vc, 16)) return pa::fail(PA_ERR_INVALID, "%s: caches must be 16-byte aligned", fn);
  if (num_blocks <= 0) return pa::fail(PA_ERR_INVALID, "%s: num_blocks %d must be positive", fn, num_blocks);
  if (block_stride < (int64_t)block_size * row_elems || block_stride % 8 != 0)
    return pa::fail(PA_ERR_INVALID, "%s: cache_block_stride %lld must be a multiple of 8 and >= B*Hkv*D = %lld", fn,
                    (long long)block_stride, (long long)((int64_t)block_size * row_elems));
  return PA_OK;
}

int hip_status(const char* fn, int err) {
  if (err != 0) return pa::fail(PA_ERR_HIP, "%s: HIP error %d (%s)", fn, err, pa::hip_error_string(err));
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return pa::g_error.c_str(); }

int pa_slot_mapping(int64_t* slot_mapping, int32_t num_tokens, const int32_t* block_tables, int32_t bt_stride,
                    const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs, int32_t block_size,
                    void* stream) {
  pa::clear_error();
  const char* fn = "slot_mapping";
  if (num_tokens < 0 || num_seqs < 0) return pa::fail(PA_ERR_INVALID, "%s: negative count", fn);
  if (block_size < 1 || block_size > 256 || (block_size & (block_size - 1)))
    return pa::fail(PA_ERR_INVALID, "%s: block_size %d must be a power of two <= 256", fn, block_size);
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping || (num_seqs > 0 && (!block_tables || !query_start_loc || !seq_lens)))
    return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (num_seqs > 0 && bt_stride < 1) return pa::fail(PA_ERR_INVALID, "%s: bt_stride %d < 1", fn, bt_stride);
  pa::SlotArgs a{slot_mapping, num_tokens, block_tables, bt_stride, query_start_loc, seq_lens, num_seqs,
                 ilog2(block_size)};
  return hip_status(fn, pa::launch_slot_mapping(a, stream));
}

}  // extern "C"

namespace {

int reshape_impl(const char* fn, const void* key, int64_t key_row_stride, const void* value,
                 int64_t value_row_stride, void* key_cache, void* value_cache, int64_t cache_block_stride,
                 int32_t num_blocks, const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                 int32_t head_dim, int32_t block_size, bool fp8, float k_scale, float v_scale, void* stream) {
  pa::clear_error();
  if (int rc = check_heads(fn, num_kv_heads, num_kv_heads, head_dim, block_size)) return rc;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (int rc = check_cache(fn, key_cache, value_cache, cache_block_stride, num_blocks, block_size, row)) return rc;
  if (fp8 && cache_block_stride % 16)
    return pa::fail(PA_ERR_INVALID, "%s: cache_block_stride %lld must be a multiple of 16 for E4M3 caches", fn,
                    (long long)cache_block_stride);
  if (fp8 && !(k_scale > 0.f && v_scale > 0.f && k_scale < __builtin_huge_valf() && v_scale < __builtin_huge_valf()))
    return pa::fail(PA_ERR_INVALID, "%s: k_scale and v_scale must be positive and finite", fn);
  if (num_tokens < 0) return pa::fail(PA_ERR_INVALID, "%s: num_tokens %d < 0", fn, num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return pa::fail(PA_ERR_INVALID, "%s: NULL input", fn);
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 8))
    return pa::fail(PA_ERR_INVALID, "%s: key/value must be 16-byte aligned", fn);
  if (key_row_stride < row || value_row_stride < row || key_row_stride % 8 || value_row_stride % 8)
    return pa::fail(PA_ERR_INVALID, "%s: row strides must be multiples of 8 and >= Hkv*D", fn);
  pa::ReshapeArgs a{key, key_row_stride, value, value_row_stride, key_cache, value_cache, cache_block_stride,
                    (int64_t)num_blocks * block_size, slot_mapping, num_tokens, (int32_t)row, ilog2(block_size),
                    fp8 ? 1 : 0, fp8 ? 1.0f / k_scale : 1.f, fp8 ? 1.0f / v_scale : 1.f};
  return hip_status(fn, pa::launch_reshape_and_cache(a, stream));
}

}  // namespace

extern "C" {

int pa_reshape_and_cache(const void* key, int64_t key_row_stride, const void* value, int64_t value_row_stride,
                         void* key_cache, void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, void* stream) {
  return reshape_impl("reshape_and_cache", key, key_row_stride, value, value_row_stride, key_cache, value_cache,
                      cache_block_stride, num_blocks, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
                      false, 1.f, 1.f, stream);
}

int pa_reshape_and_cache_fp8(const void* key, int64_t key_row_stride, const void* value, int64_t value_row_stride,
                             void* key_cache, void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                             const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, float k_scale, float v_scale, void* stream) {
  return reshape_impl("reshape_and_cache_fp8", key, key_row_stride, value, value_row_stride, key_cache,
                      value_cache, cache_block_stride, num_blocks, slot_mapping, num_tokens, num_kv_heads, head_dim,
                      block_size, true, k_scale, v_scale, stream);
}

int pa_decode_append(const void* key, int64_t key_row_stride, const void* value, int64_t value_row_stride,
                     void* key_cache, void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                     int32_t* block_tables, int32_t bt_stride, int32_t* seq_lens, const int64_t* slots,
                     const int32_t* positions, int32_t num_rows, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, void* stream) {
  pa::clear_error();
  const char* fn = "decode_append";
  if (int rc = check_heads(fn, num_kv_heads, num_kv_heads, head_dim, block_size)) return rc;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (int rc = check_cache(fn, key_cache, value_cache, cache_block_stride, num_blocks, block_size, row)) return rc;
  if (num_rows < 0) return pa::fail(PA_ERR_INVALID, "%s: num_rows %d < 0", fn, num_rows);
  if (num_rows == 0) return PA_OK;
  if (!key || !value || !block_tables || !seq_lens || !slots || !positions)
    return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  for (int32_t i = 0; i < num_rows; ++i)
    if (slots[i] >= 0 && (positions[i] < 0 || positions[i] == INT32_MAX))
      return pa::fail(PA_ERR_INVALID, "%s: row %d has position %d", fn, i, positions[i]);
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return pa::fail(PA_ERR_INVALID, "%s: key/value must be 16-byte aligned", fn);
  if (key_row_stride < row || value_row_stride < row || key_row_stride % 8 || value_row_stride % 8)
    return pa::fail(PA_ERR_INVALID, "%s: row strides must be multiples of 8 and >= Hkv*D", fn);
  if (bt_stride < 1) return pa::fail(PA_ERR_INVALID, "%s: bt_stride %d < 1", fn, bt_stride);
  pa::AppendArgs a{key_cache, value_cache, cache_block_stride, (int64_t)num_blocks * block_size, block_tables,
                   bt_stride, seq_lens, key, key_row_stride, value, value_row_stride, (int32_t)row,
                   ilog2(block_size)};
  return hip_status(fn, pa::launch_decode_append(a, slots, positions, num_rows, stream));
}

int pa_copy_blocks(void* const* caches, int32_t n_caches, int64_t block_bytes, int64_t stride_bytes,
                   int32_t num_blocks, const int32_t* pairs, int32_t n_pairs, void* stream) {
  pa::clear_error();
  const char* fn = "copy_blocks";
  if (n_pairs < 0 || n_caches < 0) return pa::fail(PA_ERR_INVALID, "%s: negative count", fn);
  if (n_pairs == 0 || n_caches == 0) return PA_OK;
  if (!caches || !pairs) return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (block_bytes <= 0 || block_bytes % 16 || stride_bytes < block_bytes || stride_bytes % 16)
    return pa::fail(PA_ERR_INVALID, "%s: block_bytes %lld must be a positive multiple of 16 <= stride %lld", fn,
                    (long long)block_bytes, (long long)stride_bytes);
  if (num_blocks <= 0) return pa::fail(PA_ERR_INVALID, "%s: num_blocks must be positive", fn);
  for (int32_t c = 0; c < n_caches; ++c)
    if (!caches[c] || !aligned(caches[c], 16)) return pa::fail(PA_ERR_INVALID, "%s: cache %d NULL or unaligned", fn, c);
  // duplicate destinations and destinations that are also sources, found on
  // sorted copies (no per-entry allocation: this runs once per step)
  std::vector<int32_t> dsts(n_pairs), srcs(n_pairs);
  for (int32_t i = 0; i < n_pairs; ++i) {
    const int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
      return pa::fail(PA_ERR_INVALID, "%s: pair %d (%d, %d) outside [0, %d)", fn, i, s, d, num_blocks);
    dsts[i] = d;
    srcs[i] = s;
  }
  std::sort(dsts.begin(), dsts.end());
  std::sort(srcs.begin(), srcs.end());
  const auto dup = std::adjacent_find(dsts.begin(), dsts.end());
  if (dup != dsts.end()) return pa::fail(PA_ERR_INVALID, "%s: destination %d named twice", fn, *dup);
  for (size_t i = 0, j = 0; i < dsts.size() && j < srcs.size();) {
    if (dsts[i] == srcs[j])
      return pa::fail(PA_ERR_INVALID, "%s: block %d is both a source and a destination", fn, dsts[i]);
    if (dsts[i] < srcs[j]) ++i; else ++j;
  }
  return hip_status(fn, pa::launch_copy_blocks(caches, n_caches, block_bytes, stride_bytes, pairs, n_pairs, stream));
}

int pa_copy_blocks_device(void* const* caches, int32_t n_caches, int64_t block_bytes, int64_t stride_bytes,
                          int32_t num_blocks, const int32_t* pairs, int32_t n_pairs, void* stream) {
  pa::clear_error();
  const char* fn = "copy_blocks_device";
  if (n_pairs < 0 || n_caches < 0) return pa::fail(PA_ERR_INVALID, "%s: negative count", fn);
  if (n_pairs == 0 || n_caches == 0) return PA_OK;
  if (!caches || !pairs) return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(pairs, 4)) return pa::fail(PA_ERR_INVALID, "%s: pairs must be 4-byte aligned", fn);
  if (block_bytes <= 0 || block_bytes % 16 || stride_bytes < block_bytes || stride_bytes % 16)
    return pa::fail(PA_ERR_INVALID, "%s: block_bytes %lld must be a positive multiple of 16 <= stride %lld", fn,
                    (long long)block_bytes, (long long)stride_bytes);
  if (num_blocks <= 0) return pa::fail(PA_ERR_INVALID, "%s: num_blocks must be positive", fn);
  for (int32_t c = 0; c < n_caches; ++c)
    if (!caches[c] || !aligned(caches[c], 16)) return pa::fail(PA_ERR_INVALID, "%s: cache %d NULL or unaligned", fn, c);
  return hip_status(fn, pa::launch_copy_blocks_device(caches, n_caches, block_bytes, stride_bytes, num_blocks, pairs,
                                                      n_pairs, stream));
}

size_t pa_paged_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                                      int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len <= 0 || partition_size <= 0) return 0;
  const int64_t parts = ((int64_t)max_seq_len + partition_size - 1) / partition_size;
  if (parts <= 1) return 0;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * parts;
  const int64_t out_bytes = ((rows * head_dim * 4) + 255) / 256 * 256;
  return (size_t)(out_bytes + rows * 4);
}

}  // extern "C"

namespace {

// The new tokens of an appending decode (all NULL for a plain one).
struct NewTokens {
  const void* key = nullptr;
  int64_t key_row_stride = 0;
  const void* value = nullptr;
  int64_t value_row_stride = 0;
  const int64_t* slots = nullptr;
  const int32_t* positions = nullptr;
};

// Validate a decode call's arguments and fill `a` (a.num_seqs = 0: nothing
// to launch).
int make_decode_args(const char* fn, void* out, float* lse, const void* q, const void* key_cache,
                     const void* value_cache, int64_t cache_block_stride, int32_t num_blocks,
                     const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t max_seq_len, int32_t partition_size, float scale, bool fp8, float k_scale, float v_scale,
                     void* workspace, size_t workspace_bytes, const NewTokens& nt, pa::DecodeArgs& a) {
  a = pa::DecodeArgs{};
  if (int rc = check_heads(fn, num_q_heads, num_kv_heads, head_dim, block_size)) return rc;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (int rc = check_cache(fn, key_cache, value_cache, cache_block_stride, num_blocks, block_size, row)) return rc;
  if (fp8 && cache_block_stride % 16)
    return pa::fail(PA_ERR_INVALID, "%s: cache_block_stride %lld must be a multiple of 16 for E4M3 caches", fn,
                    (long long)cache_block_stride);
  if (fp8 && !(k_scale > 0.f && v_scale > 0.f && k_scale < __builtin_huge_valf() && v_scale < __builtin_huge_valf()))
    return pa::fail(PA_ERR_INVALID, "%s: k_scale and v_scale must be positive and finite", fn);
  if (num_seqs < 0) return pa::fail(PA_ERR_INVALID, "%s: num_seqs < 0", fn);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !block_tables || !seq_lens) return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(out, 16) || !aligned(q, 16) || (lse && !aligned(lse, 4)))
    return pa::fail(PA_ERR_INVALID, "%s: q/out must be 16-byte aligned", fn);
  if (max_seq_len <= 0) return pa::fail(PA_ERR_INVALID, "%s: max_seq_len must be positive", fn);
  if (((int64_t)max_seq_len + block_size - 1) / block_size > bt_stride)
    return pa::fail(PA_ERR_INVALID, "%s: ceil(max_seq_len / B) exceeds bt_stride %d", fn, bt_stride);
  if (partition_size < 0 || (partition_size > 0 && (partition_size % 64 || partition_size % block_size)))
    return pa::fail(PA_ERR_INVALID, "%s: partition_size %d must be 0 or a multiple of 64 and of B", fn,
                    partition_size);
  if (!(scale == scale)) return pa::fail(PA_ERR_INVALID, "%s: scale is NaN", fn);
  int32_t P = partition_size;
  if (P == 0 || P >= max_seq_len) P = (int32_t)(((int64_t)max_seq_len + 63) / 64 * 64);
  const int64_t parts = ((int64_t)max_seq_len + P - 1) / P;
  const size_t need = pa_paged_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len, P);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return pa::fail(PA_ERR_INVALID, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
  if (parts > 65535) return pa::fail(PA_ERR_INVALID, "%s: too many partitions (%lld)", fn, (long long)parts);
  const bool append = nt.slots != nullptr;
  if (append) {
    if (!nt.key || !nt.value || !nt.positions) return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
    if (!aligned(nt.key, 16) || !aligned(nt.value, 16))
      return pa::fail(PA_ERR_INVALID, "%s: key/value must be 16-byte aligned", fn);
    if (nt.key_row_stride < row || nt.value_row_stride < row || nt.key_row_stride % 8 || nt.value_row_stride % 8)
      return pa::fail(PA_ERR_INVALID, "%s: row strides must be multiples of 8 and >= Hkv*D", fn);
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    for (int32_t i = 0; i < num_seqs; ++i) {
      if (nt.slots[i] < 0) continue;
      if (nt.slots[i] >= num_slots)
        return pa::fail(PA_ERR_INVALID, "%s: row %d has slot %lld past the pool", fn, i, (long long)nt.slots[i]);
      if (nt.positions[i] < 0 || nt.positions[i] >= max_seq_len)
        return pa::fail(PA_ERR_INVALID, "%s: row %d has position %d outside [0, max_seq_len)", fn, i,
                        nt.positions[i]);
    }
  }
  a.out = out;
  a.lse = lse;
  a.q = q;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.cache_block_stride = cache_block_stride;
  a.num_blocks = num_blocks;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.log2_block_size = ilog2(block_size);
  a.max_seq_len = max_seq_len;
  a.partition_size = P;
  a.max_parts = (int32_t)parts;
  a.scale = fp8 ? scale * k_scale : scale;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.fp8 = fp8 ? 1 : 0;
  // Explicit partitions with head_dim 128 and a multiple of 4 KV heads take
  // the row layout, whose waves read whole token rows of 4 heads: bf16
  // caches up to 1024 tokens per partition, E4M3 caches up to 512 and with
  // at most 4 query heads per KV head (one wave's item holds half the bytes
  // of a bf16 one, so longer partitions leave too few items in flight); the
  // rest the head layout.
  a.rows = (head_dim == 128 && num_kv_heads % 4 == 0 && partition_size > 0 &&
            (fp8 ? partition_size <= 512 && num_q_heads / num_kv_heads <= 4 : partition_size <= 1024))
               ? 1
               : 0;
  if (parts > 1) {
    const int64_t rows = (int64_t)num_seqs * num_q_heads * parts;
    a.ws_out = static_cast<float*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((rows * head_dim * 4) + 255) / 256 * 256);
  }
  if (append) {
    a.new_key = nt.key;
    a.new_key_stride = nt.key_row_stride;
    a.new_value = nt.value;
    a.new_value_stride = nt.value_row_stride;
    a.wr_tables = const_cast<int32_t*>(block_tables);
    a.wr_lens = const_cast<int32_t*>(seq_lens);
  }
  return PA_OK;
}

int decode_impl(const char* fn, void* out, float* lse, const void* q, const void* key_cache,
                const void* value_cache, int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables,
                int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                int32_t partition_size, float scale, bool fp8, float k_scale, float v_scale, void* workspace,
                size_t workspace_bytes, void* stream, const NewTokens& nt = NewTokens()) {
  pa::clear_error();
  pa::DecodeArgs a;
  if (int rc = make_decode_args(fn, out, lse, q, key_cache, value_cache, cache_block_stride, num_blocks, block_tables,
                                bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_seq_len, partition_size, scale, fp8, k_scale, v_scale, workspace, workspace_bytes,
                                nt, a))
    return rc;
  if (a.num_seqs == 0) return PA_OK;
  if (nt.slots) return hip_status(fn, pa::launch_paged_decode_append(a, nt.slots, nt.positions, stream));
  return hip_status(fn, pa::launch_paged_decode(a, stream));
}

}  // namespace

extern "C" {

int pa_paged_decode(void* out, float* lse, const void* q, const void* key_cache, const void* value_cache,
                    int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_seq_len, int32_t partition_size, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl("paged_decode", out, lse, q, key_cache, value_cache, cache_block_stride, num_blocks,
                     block_tables, bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_seq_len, partition_size, scale, false, 1.f, 1.f, workspace, workspace_bytes, stream);
}

int pa_paged_decode_noalloc(void* out, float* lse, const void* q, const void* key_cache, const void* value_cache,
                            int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables,
                            int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                            int32_t partition_size, float scale, void* stream) {
  static_assert(pa::kStaticScratchBytes == PA_STATIC_SCRATCH_BYTES, "scratch size differs from the header's");
  const char* fn = "paged_decode_noalloc";
  pa::clear_error();
  const size_t need = num_seqs > 0 && partition_size > 0
                          ? pa_paged_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len,
                                                           partition_size)
                          : 0;
  if (need > pa::kStaticScratchBytes)
    return pa::fail(PA_ERR_INVALID,
                    "%s: the call needs %zu bytes of split-K partials, more than the %zu-byte static scratch "
                    "(use a larger partition_size, or pa_paged_decode with a workspace)",
                    fn, need, pa::kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0)
    if (int e = pa::static_decode_scratch(&ws)) return hip_status(fn, e);
  return decode_impl(fn, out, lse, q, key_cache, value_cache, cache_block_stride, num_blocks, block_tables, bt_stride,
                     seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len, partition_size,
                     scale, false, 1.f, 1.f, ws, need > 0 ? pa::kStaticScratchBytes : 0, stream);
}

int pa_paged_decode_append(void* out, float* lse, const void* q, void* key_cache, void* value_cache,
                           int64_t cache_block_stride, int32_t num_blocks, int32_t* block_tables, int32_t bt_stride,
                           int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_seq_len, int32_t partition_size,
                           float scale, const void* key, int64_t key_row_stride, const void* value,
                           int64_t value_row_stride, const int64_t* slots, const int32_t* positions, void* workspace,
                           size_t workspace_bytes, void* stream) {
  NewTokens nt;
  nt.key = key;
  nt.key_row_stride = key_row_stride;
  nt.value = value;
  nt.value_row_stride = value_row_stride;
  nt.slots = slots;
  nt.positions = positions;
  if (num_seqs > 0 && !slots) {
    pa::clear_error();
    return pa::fail(PA_ERR_INVALID, "paged_decode_append: NULL argument");
  }
  return decode_impl("paged_decode_append", out, lse, q, key_cache, value_cache, cache_block_stride, num_blocks,
                     block_tables, bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_seq_len, partition_size, scale, false, 1.f, 1.f, workspace, workspace_bytes, stream, nt);
}

int pa_paged_decode_fp8(void* out, float* lse, const void* q, const void* key_cache, const void* value_cache,
                        int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables,
                        int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                        int32_t partition_size, float scale, float k_scale, float v_scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return decode_impl("paged_decode_fp8", out, lse, q, key_cache, value_cache, cache_block_stride, num_blocks,
                     block_tables, bt_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_seq_len, partition_size, scale, true, k_scale, v_scale, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Validate a prefill call's arguments and fill `a` (a.num_seqs = 0: nothing
// to launch).
int make_prefill_args(const char* fn, void* out, const void* q, const void* key_cache, const void* value_cache,
                      int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                      const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, float scale, int32_t causal, bool fp8, float k_scale,
                      float v_scale, pa::PrefillArgs& a) {
  a = pa::PrefillArgs{};
  if (int rc = check_heads(fn, num_q_heads, num_kv_heads, head_dim, block_size)) return rc;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (int rc = check_cache(fn, key_cache, value_cache, cache_block_stride, num_blocks, block_size, row)) return rc;
  if (fp8 && cache_block_stride % 16)
    return pa::fail(PA_ERR_INVALID, "%s: cache_block_stride %lld must be a multiple of 16 for E4M3 caches", fn,
                    (long long)cache_block_stride);
  if (fp8 && !(k_scale > 0.f && v_scale > 0.f && k_scale < __builtin_huge_valf() && v_scale < __builtin_huge_valf()))
    return pa::fail(PA_ERR_INVALID, "%s: k_scale and v_scale must be positive and finite", fn);
  if (num_seqs < 0 || max_query_len < 0) return pa::fail(PA_ERR_INVALID, "%s: negative size", fn);
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !block_tables || !query_start_loc || !seq_lens)
    return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(out, 16) || !aligned(q, 16)) return pa::fail(PA_ERR_INVALID, "%s: q/out must be 16-byte aligned", fn);
  if (max_seq_len <= 0 || max_query_len > max_seq_len)
    return pa::fail(PA_ERR_INVALID, "%s: need 0 < max_query_len <= max_seq_len", fn);
  if (((int64_t)max_seq_len + block_size - 1) / block_size > bt_stride)
    return pa::fail(PA_ERR_INVALID, "%s: ceil(max_seq_len / B) exceeds bt_stride %d", fn, bt_stride);
  if (!(scale == scale)) return pa::fail(PA_ERR_INVALID, "%s: scale is NaN", fn);
  a.out = out;
  a.q = q;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.cache_block_stride = cache_block_stride;
  a.num_blocks = num_blocks;
  a.block_tables = block_tables;
  a.bt_stride = bt_stride;
  a.query_start_loc = query_start_loc;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.max_query_len = max_query_len;
  a.max_seq_len = max_seq_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.log2_block_size = ilog2(block_size);
  a.scale = fp8 ? scale * k_scale : scale;
  a.causal = causal;
  a.fp8 = fp8 ? 1 : 0;
  a.v_scale = fp8 ? v_scale : 1.f;
  return PA_OK;
}

int prefill_impl(const char* fn, void* out, const void* q, const void* key_cache, const void* value_cache,
                 int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                 const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs, int32_t max_query_len,
                 int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, float scale, int32_t causal, bool fp8, float k_scale, float v_scale,
                 void* stream) {
  pa::clear_error();
  pa::PrefillArgs a;
  if (int rc = make_prefill_args(fn, out, q, key_cache, value_cache, cache_block_stride, num_blocks, block_tables,
                                 bt_stride, query_start_loc, seq_lens, num_seqs, max_query_len, max_seq_len,
                                 num_q_heads, num_kv_heads, head_dim, block_size, scale, causal, fp8, k_scale,
                                 v_scale, a))
    return rc;
  if (a.num_seqs == 0) return PA_OK;
  return hip_status(fn, pa::launch_paged_prefill(a, stream));
}

// Requests 0 .. n - 1 with one query each (the decode rows of a mixed batch):
// the leading run of query_start_loc_host steps of 1.  -1 if
// query_start_loc_host is not a non-decreasing sequence from 0.
int32_t leading_decodes(const int32_t* qsl, int32_t num_seqs) {
  if (qsl[0] != 0) return -1;
  int32_t n = 0;
  bool run = true;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t ql = qsl[i + 1] - qsl[i];
    if (ql < 0) return -1;
    if (run && ql == 1)
      ++n;
    else
      run = false;
  }
  return n;
}

}  // namespace

extern "C" {

int pa_paged_prefill(void* out, const void* q, const void* key_cache, const void* value_cache,
                     int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                     const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs, int32_t max_query_len,
                     int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, float scale, int32_t causal, void* stream) {
  return prefill_impl("paged_prefill", out, q, key_cache, value_cache, cache_block_stride, num_blocks, block_tables,
                      bt_stride, query_start_loc, seq_lens, num_seqs, max_query_len, max_seq_len, num_q_heads,
                      num_kv_heads, head_dim, block_size, scale, causal, false, 1.f, 1.f, stream);
}

int pa_paged_prefill_fp8(void* out, const void* q, const void* key_cache, const void* value_cache,
                         int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables,
                         int32_t bt_stride, const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, float scale, float k_scale, float v_scale,
                         int32_t causal, void* stream) {
  return prefill_impl("paged_prefill_fp8", out, q, key_cache, value_cache, cache_block_stride, num_blocks,
                      block_tables, bt_stride, query_start_loc, seq_lens, num_seqs, max_query_len, max_seq_len,
                      num_q_heads, num_kv_heads, head_dim, block_size, scale, causal, true, k_scale, v_scale, stream);
}

}  // extern "C"

extern "C" {

size_t pa_paged_attention_workspace_size(const int32_t* query_start_loc_host, int32_t num_seqs, int32_t num_q_heads,
                                         int32_t head_dim, int32_t max_seq_len, int32_t partition_size) {
  if (!query_start_loc_host || num_seqs <= 0) return 0;
  const int32_t nd = leading_decodes(query_start_loc_host, num_seqs);
  return nd > 0 ? pa_paged_decode_workspace_size(nd, num_q_heads, head_dim, max_seq_len, partition_size) : 0;
}

int pa_paged_attention(void* out, const void* q, const void* key_cache, const void* value_cache,
                       int64_t cache_block_stride, int32_t num_blocks, const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* query_start_loc, const int32_t* query_start_loc_host, const int32_t* seq_lens,
                       int32_t num_seqs, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t partition_size,
                       float scale, int32_t causal, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "paged_attention";
  pa::clear_error();
  if (num_seqs < 0) return pa::fail(PA_ERR_INVALID, "%s: num_seqs < 0", fn);
  if (num_seqs == 0) return PA_OK;
  if (!query_start_loc_host || !query_start_loc || !block_tables || !seq_lens)
    return pa::fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  const int32_t nd = leading_decodes(query_start_loc_host, num_seqs);
  if (nd < 0)
    return pa::fail(PA_ERR_INVALID, "%s: query_start_loc_host must start at 0 and not decrease", fn);
  // the prefill requests' longest query (every request's must fit max_query_len)
  int32_t pre_max_q = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t ql = query_start_loc_host[i + 1] - query_start_loc_host[i];
    if (ql > max_query_len)
      return pa::fail(PA_ERR_INVALID, "%s: request %d has %d queries, more than max_query_len %d", fn, i, ql,
                      max_query_len);
    if (i >= nd && ql > pre_max_q) pre_max_q = ql;
  }
  if (bt_stride < 1) return pa::fail(PA_ERR_INVALID, "%s: bt_stride must be positive", fn);
  pa::DecodeArgs d;
  if (int rc = make_decode_args(fn, out, nullptr, q, key_cache, value_cache, cache_block_stride, num_blocks,
                                block_tables, bt_stride, seq_lens, nd, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_seq_len, partition_size, scale, false, 1.f, 1.f, workspace, workspace_bytes,
                                NewTokens(), d))
    return rc;
  pa::PrefillArgs p;
  if (int rc = make_prefill_args(fn, out, q, key_cache, value_cache, cache_block_stride, num_blocks,
                                 block_tables + (int64_t)nd * bt_stride, bt_stride, query_start_loc + nd, seq_lens + nd,
                                 num_seqs - nd, pre_max_q, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                                 block_size, scale, causal, false, 1.f, 1.f, p))
    return rc;
  if (d.num_seqs == 0 && p.num_seqs == 0) return PA_OK;
  // fields the fused launch reads from the other kind's arguments
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.log2_block_size = ilog2(block_size);
  p.num_blocks = num_blocks;
  p.cache_block_stride = cache_block_stride;
  return hip_status(fn, pa::launch_paged_varlen(p, d, stream));
}

}  // extern "C"
