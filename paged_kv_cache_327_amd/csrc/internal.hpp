// Internal declarations shared by the C-ABI layer and the HIP launchers.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pa {

// Records the thread-local error text and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Launchers (defined in the .hip translation units).  They enqueue on
// `stream` and return a hipError_t value (0 on success); arguments have been
// validated by the caller.
struct ReshapeArgs {
  const void* key;
  int64_t key_row_stride;
  const void* value;
  int64_t value_row_stride;
  void* key_cache;
  void* value_cache;
  int64_t cache_block_stride;
  int64_t num_slots;  // num_blocks * block_size
  const int64_t* slot_mapping;
  int32_t num_tokens;
  int32_t row_elems;  // num_kv_heads * head_dim
  int32_t log2_block_size;
  int32_t fp8;        // caches hold E4M3 codes (1 byte per element)
  float k_recip;      // fp32(1 / k_scale), fp32(1 / v_scale) (fp8 only)
  float v_recip;
};
int launch_reshape_and_cache(const ReshapeArgs& a, void* stream);

struct AppendArgs {
  void* key_cache;
  void* value_cache;
  int64_t cache_block_stride;
  int64_t num_slots;  // num_blocks * block_size
  int32_t* block_tables;
  int32_t bt_stride;
  int32_t* seq_lens;
  const void* key;
  int64_t key_row_stride;
  const void* value;
  int64_t value_row_stride;
  int32_t row_elems;  // num_kv_heads * head_dim
  int32_t log2_block_size;
};
// slots, positions: host arrays of num_rows entries (they travel in the
// kernel arguments)
int launch_decode_append(const AppendArgs& a, const int64_t* slots, const int32_t* positions, int32_t num_rows,
                         void* stream);

struct SlotArgs {
  int64_t* slot_mapping;
  int32_t num_tokens;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  int32_t num_seqs;
  int32_t log2_block_size;
};
int launch_slot_mapping(const SlotArgs& a, void* stream);

int launch_copy_blocks(void* const* caches, int32_t n_caches, int64_t block_bytes,
                       int64_t stride_bytes, const int32_t* pairs, int32_t n_pairs,
                       void* stream);
// pairs: device int32 [n_pairs][2]; pairs with an id outside [0, num_blocks)
// are skipped
int launch_copy_blocks_device(void* const* caches, int32_t n_caches, int64_t block_bytes, int64_t stride_bytes,
                              int32_t num_blocks, const int32_t* pairs, int32_t n_pairs, void* stream);

// The fields the decode prologue's first loads need come first, so that the
// kernel reads them with its first argument loads.
struct DecodeArgs {
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const void* q;
  int32_t bt_stride;
  int32_t log2_block_size;
  int32_t max_seq_len;
  int32_t partition_size;  // > 0, multiple of 64 and of the block size
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  void* out;
  float* lse;
  const void* key_cache;
  const void* value_cache;
  int64_t cache_block_stride;
  int32_t num_blocks;
  int32_t max_parts;
  float scale;     // softmax scale (times k_scale for E4M3 caches)
  float v_scale;   // 1 for bf16 caches
  int32_t fp8;     // caches hold E4M3 codes (1 byte per element)
  int32_t rows;    // row layout: a wave per (4 KV heads, partition, sequence)
  float* ws_out;  // [S][Hq][max_parts][D]   (max_parts > 1 only)
  float* ws_lse;  // [S][Hq][max_parts]
  // appending decode only: the new tokens' K/V rows and the writable tables
  // and lengths (the same arrays as block_tables and seq_lens)
  const void* new_key;
  int64_t new_key_stride;
  const void* new_value;
  int64_t new_value_stride;
  int32_t* wr_tables;
  int32_t* wr_lens;
};
int launch_paged_decode(const DecodeArgs& a, void* stream);
// The allocation-free entry point's scratch: its device address on the
// current GPU (looked up once per device), kStaticScratchBytes long.
constexpr size_t kStaticScratchBytes = size_t{64} << 20;
int static_decode_scratch(void** ptr);
// slots, positions: host arrays of num_seqs entries (kernel arguments)
int launch_paged_decode_append(const DecodeArgs& a, const int64_t* slots, const int32_t* positions, void* stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* key_cache;
  const void* value_cache;
  int64_t cache_block_stride;
  int32_t num_blocks;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  int32_t num_seqs, max_query_len, max_seq_len;
  int32_t num_q_heads, num_kv_heads, head_dim;
  int32_t log2_block_size;
  float scale;     // softmax scale (times k_scale for E4M3 caches)
  int32_t causal;
  int32_t fp8;     // caches hold E4M3 codes (1 byte per element)
  float v_scale;   // 1 for bf16 caches
};
int launch_paged_prefill(const PrefillArgs& a, void* stream);
// Work-groups of a prefill launch (0 when a.num_seqs is 0; -1 when too many).
int64_t prefill_grid_size(const PrefillArgs& a);
// The decode's log-sum-exp merge pass alone (nothing when a.max_parts <= 1).
int launch_decode_merge(const DecodeArgs& a, void* stream);
// A mixed batch in one launch: prefill requests p and decode rows d (either
// may have num_seqs 0), then the decode rows' merge pass.
int launch_paged_varlen(const PrefillArgs& p, const DecodeArgs& d, void* stream);

const char* hip_error_string(int err);

}  // namespace pa
