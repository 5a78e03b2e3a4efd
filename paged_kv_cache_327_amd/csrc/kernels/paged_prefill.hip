// Chunked-prefill attention over a paged KV cache on gfx950 MFMA.
//
// What is computed ("PagedAttention: fragmentation, blocks, block tables",
// attention-metadata section): request i's queries are rows
// query_start_loc[i] .. query_start_loc[i+1]-1 and are the last q_i of its
// seq_lens[i] tokens; query j (absolute position c_i + j) attends to the keys
// 0 .. c_i + j (causal) gathered through row i of the block table.  The
// kernel design below is ours; the pages give none.
//
// Work-group = 4 waves = (request i, a group of HW query heads sharing one KV
// head, a tile of 32 * (4 / HW) queries).  Each wave owns one head and 32
// queries.  Key tiles of 64 keys are gathered through the block table into
// LDS once per work-group and used by all of its waves (the GQA sharing):
//   * K and V are stored row-major [key][d] with the 16-byte chunks of each
//     row permuted (an XOR with a function of the row), which keeps both the
//     S^T operand reads and the transposing V^T reads (gfx950's
//     ds_read_b64_tr_b16) free of bank conflicts without padding.  Loads of
//     keys past the sequence end are redirected to a written row and those
//     keys are masked out of the softmax, so bytes of unwritten slots (NaN,
//     say) can never reach a product.
//   * bf16 caches go from HBM straight into LDS (global_load_lds_dwordx4:
//     lane l of a wave writes bytes 16 l .. 16 l + 15 of a 1 KiB window, so
//     each lane fetches the chunk that the permuted layout puts there); no
//     register holds a staged tile.  E4M3 codes are staged in registers and
//     converted to bf16 on their way into LDS.
//   * Each wave stages 16 keys of the tile.  With B >= 16 they lie in one
//     block: the block id is a scalar load and the row base a scalar address.
//     With B < 16 every key has its own block; when a cache's whole byte
//     span fits in 32 bits the lanes' offsets are 32-bit (KO 1; KO 2 with
//     B = 1, where a key's offset is its block's alone), so the loads take
//     a scalar base and a 32-bit lane offset there too.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane owns one query column,
//     so the softmax max and sum are in-lane (plus one exchange between the
//     two lane halves).
//   * P^T comes straight out of the S^T registers (rounded to bf16); the key
//     order inside each 16-key MFMA step is permuted identically on P^T and on
//     V^T, which leaves the sum unchanged and needs no data movement.
//   * O^T += V^T P^T accumulates in fp32; the online softmax raises its
//     running maximum only when a score exceeds it by more than 8 (log2
//     units), which keeps the result exact and rescales rare.
//   * The next key tile's K/V loads are in flight while the current tile is
//     computed (double-buffered LDS, one barrier per tile); block-table
//     entries are fetched one further tile ahead.
//   * bf16 caches: the leading tiles that no query of the work-group masks
//     are software-pipelined (the QK^T MFMAs of tile t + 1 issued between
//     the exponentials of tile t, the PV MFMAs of tile t beside the maximum
//     of tile t + 1), with K loaded one tile ahead of V; the masked tiles at
//     the diagonal take the plain steps.
#include <type_traits>

#include "../internal.hpp"
#include "common.hpp"
#include "prefill_body.hpp"

namespace pa {
namespace {

using namespace prefill_body;

template <int D, int HW, bool CAUSAL, bool BIG, bool F8, int KO>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PrefillArgs a) {
  prefill_tile<D, HW, CAUSAL, BIG, F8, KO>(a, blockIdx.x);
}

template <int D, int HW, bool CAUSAL, bool BIG, bool F8>
void launch_one(const PrefillArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (!BIG) {
    // B < 16: 32-bit key offsets when every byte offset of a cache fits
    // (num_blocks block strides; ids are clamped into [0, num_blocks))
    // (block size 1: a key is row 0 of its block)
    const int64_t span = (int64_t)a.num_blocks * a.cache_block_stride * (F8 ? 1 : 2);
    if (span <= 0xffffffffLL) {
      if (a.log2_block_size == 0)
        hipLaunchKernelGGL((prefill_kernel<D, HW, CAUSAL, BIG, F8, 2>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((prefill_kernel<D, HW, CAUSAL, BIG, F8, 1>), grid, dim3(256), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((prefill_kernel<D, HW, CAUSAL, BIG, F8, 0>), grid, dim3(256), 0, st, a);
}

template <int D, int HW>
int launch_hw(const PrefillArgs& a, hipStream_t st) {
  const int span = kQ * (4 / HW);
  const int64_t X = (a.max_query_len + span - 1) / span;
  const int64_t groups = (int64_t)a.num_seqs * (a.num_q_heads / HW);
  const int64_t n = X * kXcds * ((groups + kXcds - 1) / kXcds);
  if (n * 256 > 0xffffffffLL) return (int)hipErrorInvalidConfiguration;   // grid size in work-items is 32-bit
  const dim3 grid((unsigned)n);
  const bool big = a.log2_block_size >= 4;
  if (a.fp8) {
    if (a.causal && big)
      launch_one<D, HW, true, true, true>(a, grid, st);
    else if (a.causal)
      launch_one<D, HW, true, false, true>(a, grid, st);
    else if (big)
      launch_one<D, HW, false, true, true>(a, grid, st);
    else
      launch_one<D, HW, false, false, true>(a, grid, st);
  } else if (a.causal && big)
    launch_one<D, HW, true, true, false>(a, grid, st);
  else if (a.causal)
    launch_one<D, HW, true, false, false>(a, grid, st);
  else if (big)
    launch_one<D, HW, false, true, false>(a, grid, st);
  else
    launch_one<D, HW, false, false, false>(a, grid, st);
  return (int)hipGetLastError();
}

template <int D>
int launch_d(const PrefillArgs& a, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (G % 4 == 0) return launch_hw<D, 4>(a, st);
  if (G % 2 == 0) return launch_hw<D, 2>(a, st);
  return launch_hw<D, 1>(a, st);
}

}  // namespace

int64_t prefill_grid_size(const PrefillArgs& a) {
  if (a.num_seqs <= 0 || a.max_query_len <= 0) return 0;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int HW = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  const int span = kQ * (4 / HW);
  const int64_t X = (a.max_query_len + span - 1) / span;
  const int64_t groups = (int64_t)a.num_seqs * (a.num_q_heads / HW);
  const int64_t n = X * kXcds * ((groups + kXcds - 1) / kXcds);
  return n * 256 > 0xffffffffLL ? -1 : n;
}

int launch_paged_prefill(const PrefillArgs& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace pa
