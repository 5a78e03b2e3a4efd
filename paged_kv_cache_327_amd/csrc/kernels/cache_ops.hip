// Slot mapping, KV-cache write by slot mapping (bf16, or E4M3 with a
// per-cache scale) and whole-block copy-on-write copies.
//
// The write and the copy move bits with 16-byte vector loads and stores and
// are bound by HBM bandwidth; the slot mapping is integer work on a few
// thousand tokens.
#include "../internal.hpp"
#include "common.hpp"

namespace pa {
namespace {

// One wave per token: the wave reads the token's slot once (wave-uniform,
// so it is a scalar load) and copies its K and V rows (Hkv*D bf16 each) in
// 16-byte pieces.  "PagedAttention: fragmentation, blocks, block tables",
// 3. The slot mapping: the write goes to flat row slot of block-major storage,
// block slot / B at offset slot % B; the padding id (-1) writes nothing.
//
// E4M3 caches (F8): each bf16 element x is stored as the E4M3 code of the
// fp32 product x * r, r = fp32(1 / scale) of its cache ("The pantry of
// pigeonholes", knobs table: the KV cache dtype sets the bytes per element).
// A lane turns 8 bf16 (16 bytes) into 8 codes (8 bytes).
__device__ __forceinline__ uint2 quantize8(const uint4 x, float r) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = e4m3_code(__uint_as_float(w[i] << 16) * r);
    c[2 * i + 1] = e4m3_code(__uint_as_float(w[i] & 0xffff0000u) * r);
  }
  return make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24, c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
}

// A token's K and V rows, nvec 16-byte pieces each, moved by one wave: two
// pieces of each per lane are loaded before any is stored, so the loads of a
// row overlap.
__device__ __forceinline__ void copy_row(const uint4* ks, const uint4* vs, uint4* kd, uint4* vd, int nvec,
                                         int lane) {
  for (int c = lane; c < nvec; c += 128) {
    const bool two = c + 64 < nvec;
    const uint4 k0 = ks[c], v0 = vs[c];
    uint4 k1 = k0, v1 = v0;
    if (two) {
      k1 = ks[c + 64];
      v1 = vs[c + 64];
    }
    kd[c] = k0;
    vd[c] = v0;
    if (two) {
      kd[c + 64] = k1;
      vd[c + 64] = v1;
    }
  }
}

template <bool F8>
__global__ void __launch_bounds__(256) reshape_and_cache_kernel(ReshapeArgs a) {
  // wave-uniform (SGPR), so that the per-token loads below are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.num_tokens) return;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot >> a.log2_block_size;
  const int64_t off = slot & ((int64_t{1} << a.log2_block_size) - 1);
  const int64_t dst = blk * a.cache_block_stride + off * a.row_elems;
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.key) + t * a.key_row_stride);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.value) + t * a.value_row_stride);
  const int nvec = a.row_elems >> 3;
  if constexpr (F8) {
    uint2* kd = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.key_cache) + dst);
    uint2* vd = reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.value_cache) + dst);
    for (int c = lane; c < nvec; c += 64) {
      const uint4 k = ks[c];
      const uint4 v = vs[c];
      kd[c] = quantize8(k, a.k_recip);
      vd[c] = quantize8(v, a.v_recip);
    }
  } else {
    uint4* kd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.key_cache) + dst);
    uint4* vd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.value_cache) + dst);
    copy_row(ks, vs, kd, vd, nvec, lane);
  }
}

// One decode token per row; the rows' slots and positions travel in the
// kernel arguments, so a decode step needs no host-to-device copy of
// metadata and reads nothing but the new rows.  One wave per row writes the
// token's K and V rows to its slot (as the cache write above) and, from lane
// 0, records the slot's block as the table entry of the token's position p
// and stores seq_lens[row] = p + 1.  By
// the slot formula ("PagedAttention: fragmentation, blocks, block tables",
// 3. The slot mapping) that entry is slot / B, so the device tables follow
// the host pool -- a new block, or the in-place redirect of a copied tail
// (copy-on-write section) -- without being copied.  A slot of -1 changes
// nothing; an entry past the row's width is not written.
constexpr int kAppendMax = 256;   // rows per launch

struct AppendBatch {
  int64_t slots[kAppendMax];
  int32_t pos[kAppendMax];
  int32_t row0;
  int32_t n;
};

__global__ void __launch_bounds__(256) decode_append_kernel(AppendArgs a, AppendBatch b) {
  // wave-uniform (SGPR), so that the per-token loads below are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= b.n) return;
  const int64_t slot = b.slots[r];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t row = b.row0 + r;
  const int32_t p = b.pos[r];
  const int64_t blk = slot >> a.log2_block_size;
  const int64_t off = slot & ((int64_t{1} << a.log2_block_size) - 1);
  const int64_t dst = blk * a.cache_block_stride + off * a.row_elems;
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.key) + row * a.key_row_stride);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.value) + row * a.value_row_stride);
  uint4* kd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.key_cache) + dst);
  uint4* vd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.value_cache) + dst);
  copy_row(ks, vs, kd, vd, a.row_elems >> 3, lane);
  if (lane == 0) {
    const int64_t j = p >> a.log2_block_size;
    if (p >= 0 && j < a.bt_stride) {
      a.block_tables[row * a.bt_stride + j] = (int32_t)blk;
      a.seq_lens[row] = p + 1;
    }
  }
}

// One thread per step token.  Its request is the last i with
// query_start_loc[i] <= t (binary search over the num_seqs + 1 entries; the
// loop is bounded by log2 of that count even if the entries are not sorted,
// and every index stays inside the arrays).  "PagedAttention: fragmentation,
// blocks, block tables", 3. The slot mapping: slot = table[req][pos / B] * B +
// pos % B, the padding id for tokens without a slot.
__global__ void __launch_bounds__(256) slot_mapping_kernel(SlotArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.num_tokens) return;
  int64_t slot = -1;
  if (a.num_seqs > 0 && t >= a.query_start_loc[0] && t < a.query_start_loc[a.num_seqs]) {
    int lo = 0, hi = a.num_seqs;             // query_start_loc[lo] <= t, search (lo, hi)
    while (hi - lo > 1) {
      const int mid = lo + ((hi - lo) >> 1);
      if (a.query_start_loc[mid] <= t) lo = mid; else hi = mid;
    }
    const int q0 = a.query_start_loc[lo];
    const int q = a.query_start_loc[lo + 1] - q0;
    const int64_t pos = (int64_t)a.seq_lens[lo] - q + (t - q0);
    const int64_t j = pos >> a.log2_block_size;
    if (pos >= 0 && j < a.bt_stride) {
      const int64_t blk = a.block_tables[(int64_t)lo * a.bt_stride + j];
      slot = (blk << a.log2_block_size) + (pos & ((int64_t{1} << a.log2_block_size) - 1));
    }
  }
  a.slot_mapping[t] = slot;
}

constexpr int kMaxCopyCaches = 64;
constexpr int kMaxCopyPairs = 256;
constexpr int kCopyUnroll = 4;  // 16-byte vectors per thread per pass

// Pairs and cache pointers travel in the kernel arguments (about 2.5 KiB), so
// the host's pair list needs no staging buffer; a step's copy-on-write pairs
// (up to 256) and all 64 cache tensors of a 32-layer model take one launch.
struct CopyBatch {
  char* caches[kMaxCopyCaches];
  int32_t pairs[2 * kMaxCopyPairs];
  int64_t block_bytes;
  int64_t stride_bytes;
};

// grid = (chunks per block, pairs, caches).  Each chunk is 256 threads x
// kCopyUnroll x 16 B.  No destination is a source (checked on the host), so
// the copies are independent and the order of the pairs does not matter.
// "PagedAttention: fragmentation, blocks, block tables", copy-on-write
// section: blocks[dst] = blocks[src] over the byte view of every cache tensor.
__global__ void __launch_bounds__(256) copy_blocks_kernel(CopyBatch b) {
  const int pair = blockIdx.y, cache = blockIdx.z;
  const int64_t src = b.pairs[2 * pair], dst = b.pairs[2 * pair + 1];
  const uint4* s = reinterpret_cast<const uint4*>(b.caches[cache] + src * b.stride_bytes);
  uint4* d = reinterpret_cast<uint4*>(b.caches[cache] + dst * b.stride_bytes);
  const int64_t nvec = b.block_bytes >> 4;
  const int64_t base = (int64_t)blockIdx.x * (256 * kCopyUnroll) + threadIdx.x;
  uint4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < nvec) v[u] = s[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < nvec) d[i] = v[u];
  }
}

// The same copy with the pairs read from device memory (so a captured launch
// can take new pairs on every replay): pair `pair` of the array, skipped when
// either id lies outside [0, num_blocks) -- -1 pads a list to a fixed count.
struct CopyDevBatch {
  char* caches[kMaxCopyCaches];
  const int32_t* pairs;
  int32_t num_blocks;
  int64_t block_bytes;
  int64_t stride_bytes;
};

__global__ void __launch_bounds__(256) copy_blocks_dev_kernel(CopyDevBatch b, int32_t pair0) {
  const int pair = pair0 + blockIdx.y, cache = blockIdx.z;
  const int32_t src = b.pairs[2 * pair], dst = b.pairs[2 * pair + 1];
  if (src < 0 || src >= b.num_blocks || dst < 0 || dst >= b.num_blocks) return;
  const uint4* s = reinterpret_cast<const uint4*>(b.caches[cache] + (int64_t)src * b.stride_bytes);
  uint4* d = reinterpret_cast<uint4*>(b.caches[cache] + (int64_t)dst * b.stride_bytes);
  const int64_t nvec = b.block_bytes >> 4;
  const int64_t base = (int64_t)blockIdx.x * (256 * kCopyUnroll) + threadIdx.x;
  uint4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < nvec) v[u] = s[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < nvec) d[i] = v[u];
  }
}

}  // namespace

int launch_copy_blocks_device(void* const* caches, int32_t n_caches, int64_t block_bytes, int64_t stride_bytes,
                              int32_t num_blocks, const int32_t* pairs, int32_t n_pairs, void* stream) {
  const int64_t nvec = block_bytes >> 4;
  const unsigned chunks = (unsigned)((nvec + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll));
  for (int32_t c0 = 0; c0 < n_caches; c0 += kMaxCopyCaches) {
    const int32_t nc = n_caches - c0 < kMaxCopyCaches ? n_caches - c0 : kMaxCopyCaches;
    CopyDevBatch b{};
    for (int32_t i = 0; i < nc; ++i) b.caches[i] = static_cast<char*>(caches[c0 + i]);
    b.pairs = pairs;
    b.num_blocks = num_blocks;
    b.block_bytes = block_bytes;
    b.stride_bytes = stride_bytes;
    for (int32_t p0 = 0; p0 < n_pairs; p0 += 65535) {
      const int32_t np = n_pairs - p0 < 65535 ? n_pairs - p0 : 65535;
      hipLaunchKernelGGL(copy_blocks_dev_kernel, dim3(chunks, (unsigned)np, (unsigned)nc), dim3(256), 0,
                         (hipStream_t)stream, b, p0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return (int)e;
    }
  }
  return 0;
}

int launch_reshape_and_cache(const ReshapeArgs& a, void* stream) {
  const unsigned grid = (unsigned)((a.num_tokens + 3) / 4);
  if (a.fp8)
    hipLaunchKernelGGL(reshape_and_cache_kernel<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_decode_append(const AppendArgs& a, const int64_t* slots, const int32_t* positions, int32_t num_rows,
                         void* stream) {
  for (int32_t r0 = 0; r0 < num_rows; r0 += kAppendMax) {
    AppendBatch b{};
    b.row0 = r0;
    b.n = num_rows - r0 < kAppendMax ? num_rows - r0 : kAppendMax;
    for (int32_t i = 0; i < b.n; ++i) {
      b.slots[i] = slots[r0 + i];
      b.pos[i] = positions[r0 + i];
    }
    hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)((b.n + 3) / 4)), dim3(256), 0, (hipStream_t)stream, a, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

int launch_slot_mapping(const SlotArgs& a, void* stream) {
  const unsigned grid = (unsigned)((a.num_tokens + 255) / 256);
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_copy_blocks(void* const* caches, int32_t n_caches, int64_t block_bytes, int64_t stride_bytes,
                       const int32_t* pairs, int32_t n_pairs, void* stream) {
  const int64_t nvec = block_bytes >> 4;
  const unsigned chunks = (unsigned)((nvec + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll));
  for (int32_t c0 = 0; c0 < n_caches; c0 += kMaxCopyCaches) {
    const int32_t nc = n_caches - c0 < kMaxCopyCaches ? n_caches - c0 : kMaxCopyCaches;
    for (int32_t p0 = 0; p0 < n_pairs; p0 += kMaxCopyPairs) {
      const int32_t np = n_pairs - p0 < kMaxCopyPairs ? n_pairs - p0 : kMaxCopyPairs;
      CopyBatch b{};
      for (int32_t i = 0; i < nc; ++i) b.caches[i] = static_cast<char*>(caches[c0 + i]);
      for (int32_t i = 0; i < 2 * np; ++i) b.pairs[i] = pairs[2 * p0 + i];
      b.block_bytes = block_bytes;
      b.stride_bytes = stride_bytes;
      hipLaunchKernelGGL(copy_blocks_kernel, dim3(chunks, (unsigned)np, (unsigned)nc), dim3(256), 0,
                         (hipStream_t)stream, b);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return (int)e;
    }
  }
  return 0;
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace pa
