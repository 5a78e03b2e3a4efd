// A whole step's attention in one launch: the prefill chunks and the decode
// rows of a mixed batch together.
//
// What is computed ("PagedAttention: fragmentation, blocks, block tables",
// attention-metadata section): one metadata set -- query_start_loc, seq_lens
// and the block table -- describes every request of the step, and a decode
// is a request with one query.  Each request's queries attend, causally, to
// its keys gathered through its table row; the results are those of the
// chunked-prefill and decode calls.
//
// Design (ours): the grid holds the prefill work-groups of the chunked
// prefill kernel (MFMA-bound) and the partition work-groups of the decode
// kernel (HBM-bound), and each work-group runs the body of its kind, so the
// two kinds share the compute units instead of taking turns: a CU runs the
// tensor-core work of one while the other waits for memory.  The grid is cut
// into chunks of 8 consecutive work-groups, one per XCD (work-groups are
// dealt to the 8 XCDs round-robin), and the chunks are dealt to the two
// kinds in proportion, evenly through the grid; within its kind a
// work-group keeps the index it would have in its own kernel, so the
// prefill's XCD placement (all query tiles of one request and head group on
// one XCD) and its heaviest-first order hold.  Decode rows with several
// partitions are merged afterwards by the decode's merge pass.
#include "../internal.hpp"
#include "common.hpp"
#include "decode_body.hpp"
#include "prefill_body.hpp"

namespace pa {
namespace {

struct VarlenGrid {
  int32_t n_chunks;      // chunks of 8 work-groups in the grid
  int32_t n_pre_chunks;  // chunks running prefill work-groups
  int32_t dec_wgs;       // decode work-groups: max_parts x num_kv_heads x decode rows
                         // (row layout: a quarter of the wave items, rounded up)
  int32_t dec_items;     // row layout: wave items, max_parts x num_kv_heads / 4 x decode rows
};

template <int D, int G, int HW, bool CAUSAL, bool BIG, int KO, bool ROWS>
__global__ void __launch_bounds__(256, 2) varlen_kernel(PrefillArgs p, DecodeArgs d, VarlenGrid vg) {
  const int c = blockIdx.x >> 3, x = blockIdx.x & 7;
  // chunk c runs prefill when the even spread of n_pre_chunks over n_chunks
  // steps at c; kp = prefill chunks before it
  const int kp = (int)((int64_t)c * vg.n_pre_chunks / vg.n_chunks);
  const int kp1 = (int)((int64_t)(c + 1) * vg.n_pre_chunks / vg.n_chunks);
  if (kp1 > kp) {
    prefill_body::prefill_tile<D, HW, CAUSAL, BIG, false, KO>(p, 8 * kp + x);
  } else {
    const int v = 8 * (c - kp) + x;   // decode work-group, in the order of its own grid
    if (v >= vg.dec_wgs) return;
    if constexpr (ROWS) {
      const int item = 4 * v + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      if (item >= vg.dec_items) return;
      const int hsn = d.num_kv_heads >> 2;
      const int hs = item % hsn, rest = item / hsn;
      decode_body::decode_rows<G, BIG, false, decode_body::kRowBuffers<G>>(d, decode_body::NoAppend{0},
                                                                          rest % d.max_parts, hs, rest / d.max_parts);
    } else {
      const int part = v % d.max_parts, rest = v / d.max_parts;
      decode_body::decode_partition<D, G, BIG, false, false, 4>(d, decode_body::NoAppend{0}, part,
                                                               rest % d.num_kv_heads, rest / d.num_kv_heads);
    }
  }
}

template <int D, int G, bool CAUSAL, bool BIG, int KO, bool ROWS = false>
void launch_one(const PrefillArgs& p, const DecodeArgs& d, const VarlenGrid& vg, hipStream_t st) {
  constexpr int HW = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  hipLaunchKernelGGL((varlen_kernel<D, G, HW, CAUSAL, BIG, KO, ROWS>), dim3((unsigned)vg.n_chunks * 8), dim3(256),
                     0, st, p, d, vg);
}

// The decode rows in the row layout when the decode arguments chose it
// (head_dim 128 only).
template <int D, int G, bool CAUSAL, bool BIG, int KO>
void launch_layout(const PrefillArgs& p, const DecodeArgs& d, const VarlenGrid& vg, hipStream_t st) {
  if constexpr (D == 128) {
    if (d.rows) return launch_one<D, G, CAUSAL, BIG, KO, true>(p, d, vg, st);
  }
  launch_one<D, G, CAUSAL, BIG, KO>(p, d, vg, st);
}

template <int D, int G>
void launch_g(const PrefillArgs& p, const DecodeArgs& d, const VarlenGrid& vg, hipStream_t st) {
  const bool big = p.log2_block_size >= 4;
  // B < 16: 32-bit key offsets in the prefill when a cache's byte span fits
  // (block size 1: a key is row 0 of its block)
  const bool small = (int64_t)p.num_blocks * p.cache_block_stride * 2 <= 0xffffffffLL;
  const bool b1 = p.log2_block_size == 0;
  if (p.causal) {
    if (big)
      launch_layout<D, G, true, true, 0>(p, d, vg, st);
    else if (small && b1)
      launch_layout<D, G, true, false, 2>(p, d, vg, st);
    else if (small)
      launch_layout<D, G, true, false, 1>(p, d, vg, st);
    else
      launch_layout<D, G, true, false, 0>(p, d, vg, st);
  } else {
    if (big)
      launch_layout<D, G, false, true, 0>(p, d, vg, st);
    else if (small && b1)
      launch_layout<D, G, false, false, 2>(p, d, vg, st);
    else if (small)
      launch_layout<D, G, false, false, 1>(p, d, vg, st);
    else
      launch_layout<D, G, false, false, 0>(p, d, vg, st);
  }
}

// Head ratios whose two bodies fit one work-group's registers (two waves per
// SIMD, no spills to AGPRs): at head_dim 128 up to 5 query heads per KV head.
constexpr int kMaxFusedG128 = 5;

template <int D>
void launch_d(const PrefillArgs& p, const DecodeArgs& d, const VarlenGrid& vg, hipStream_t st) {
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: return launch_g<D, 1>(p, d, vg, st);
    case 2: return launch_g<D, 2>(p, d, vg, st);
    case 3: return launch_g<D, 3>(p, d, vg, st);
    case 4: return launch_g<D, 4>(p, d, vg, st);
    case 5: return launch_g<D, 5>(p, d, vg, st);
  }
  if constexpr (D == 64) {
    switch (p.num_q_heads / p.num_kv_heads) {
      case 6: return launch_g<D, 6>(p, d, vg, st);
      case 7: return launch_g<D, 7>(p, d, vg, st);
      case 8: return launch_g<D, 8>(p, d, vg, st);
    }
  }
}

}  // namespace

int launch_paged_varlen(const PrefillArgs& p, const DecodeArgs& d, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  if (p.head_dim == 128 && p.num_q_heads / p.num_kv_heads > kMaxFusedG128) {
    // the two kinds' kernels one after the other on the stream
    if (p.num_seqs > 0)
      if (int e = launch_paged_prefill(p, stream)) return e;
    return d.num_seqs > 0 ? launch_paged_decode(d, stream) : 0;
  }
  const int64_t n_pre = prefill_grid_size(p);
  if (n_pre < 0) return (int)hipErrorInvalidConfiguration;
  int64_t dec = 0, dec_items = 0;
  if (d.num_seqs > 0 && d.rows) {
    dec_items = (int64_t)d.max_parts * (d.num_kv_heads / 4) * d.num_seqs;
    dec = (dec_items + 3) / 4;
  } else if (d.num_seqs > 0) {
    dec = (int64_t)d.max_parts * d.num_kv_heads * d.num_seqs;
  }
  const int64_t chunks = n_pre / 8 + (dec + 7) / 8;
  if (chunks == 0) return 0;
  if (chunks * 8 * 256 > 0xffffffffLL) return (int)hipErrorInvalidConfiguration;
  VarlenGrid vg;
  vg.n_chunks = (int32_t)chunks;
  vg.n_pre_chunks = (int32_t)(n_pre / 8);
  vg.dec_wgs = (int32_t)dec;
  vg.dec_items = (int32_t)dec_items;
  if (p.head_dim == 64)
    launch_d<64>(p, d, vg, st);
  else
    launch_d<128>(p, d, vg, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  return d.num_seqs > 0 ? launch_decode_merge(d, stream) : 0;
}

}  // namespace pa
