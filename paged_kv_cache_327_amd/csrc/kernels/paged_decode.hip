// Paged decode attention for gfx950: a split-K partition pass plus a
// log-sum-exp merge.
//
// What is computed ("PagedAttention: fragmentation, blocks, block tables",
// attention-metadata section; "The pantry of pigeonholes", "The mechanism"):
// for sequence s, the kernel walks row s of the block table in logical order
// for ceil(seq_lens[s] / B) entries and attends one query per head over the
// gathered K/V.  The first page names splitting a sequence's keys across
// work-groups (split-K) among the kernel's concerns but gives no design; the
// design below is ours.
//
// Partition pass: one work-group per (partition, KV head g, seq s), of 4
// waves (8 for E4M3 caches with at most 4 query heads per KV head, whose
// registers allow four waves per SIMD).
//  * A token's K (or V) row of head g is held by D / 8 lanes, 8 elements
//    each (one 16-byte piece of bf16, or 8 one-byte E4M3 codes), so every
//    row load is a coalesced access of the row's contiguous bytes.  With
//    D = 128 a wave's four 16-lane rows hold 4 consecutive tokens per load
//    instruction, with D = 64 its eight 8-lane groups hold 8.  A wave works
//    on 16-token tiles and keeps the next tile's loads in flight while it
//    computes the current one.  Eight elements per lane keep a lane's
//    queries (G x 4 registers) and accumulators (G x 8) small enough for
//    three waves per SIMD at D = 128 and G = 4.
//  * E4M3 caches: the codes become bf16 pairs exactly
//    (v_cvt_scalef32_pk_bf16_fp8 at scale 1) and the rest is the bf16 path;
//    k_scale is folded into the logit scale and v_scale into the output.
//  * Block lookup: with B >= 16 a tile lies inside one block, whose id is a
//    scalar load from the table row and whose base address is scalar; with
//    B < 16 the partition's table entries are staged in LDS and each token
//    looks its block up there.  Ids are clamped into [0, num_blocks).
//  * The G = Hq/Hkv query heads of KV head g all use the same K/V registers
//    (the GQA sharing).  q.k partial sums (v_dot2_f32_bf16) of 4 heads x the
//    group's tokens are reduce-scattered over the group's lanes with DPP, so
//    each lane finishes one (head, token) score and takes one exponential;
//    the bf16 weights are paired over tokens and broadcast back to the group
//    with DPP, and p.v runs on token pairs with v_dot2_f32_bf16 into fp32
//    accumulators.
//  * Online softmax in log2 units with one running maximum per head shared by
//    the whole wave.  It is raised only when a score exceeds it by more than
//    8 (weights stay <= 2^8): a ballot sends the wave to a rare slow path, so
//    the fast path has no per-lane branches and the lane groups never need
//    rescaling against each other.
//  * Merge: the lane groups' sums add directly (shared maxima): the four
//    16-lane rows in registers with gfx950's lane swaps (v_permlane32_swap,
//    v_permlane16_swap), the waves through LDS with the log-sum-exp
//    identity.  A sequence with one partition writes its bf16 output
//    directly; otherwise partials (normalised output, log2 lse) go to the
//    workspace for the merge pass.
//
// Row layouts (explicit partitions, head_dim 128, a multiple of 4 KV heads):
// one wave per (set of 4 KV heads, partition, sequence), four per
// work-group, no LDS.  bf16 (partitions up to 1024 tokens): 16-lane row r
// holds KV head 4 hs + r, 8 elements per lane, so one load reads a token's
// rows of the 4 heads (1 KiB contiguous).  E4M3 (partitions up to 512, at
// most 4 query heads per KV head): 16 codes per lane, the half rows holding
// tokens of either parity, so one load reads two tokens' 512-byte runs.
// Both keep each row's running maxima in the row (one KV head per row).
//
// Merge pass: one wave per (query head, sequence) combines the partials of
// up to 64 partitions per round with the log-sum-exp identity.
#include <mutex>
#include <type_traits>

#include "../internal.hpp"
#include "common.hpp"
#include "decode_body.hpp"

namespace pa {
namespace {

using namespace decode_body;

template <int D, int G, bool BIG, bool F8, bool APP>
__global__ void __launch_bounds__((64 * kWaves<F8, G>)) decode_partition_kernel(DecodeArgs a, RowsOf<APP> rows) {
  decode_partition<D, G, BIG, F8, APP>(a, rows, blockIdx.x, blockIdx.y, (int)blockIdx.z);
}

// out[s, h] = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M) over the
// sequence's partitions (log-sum-exp identity); lse = (M + log2 W) ln 2.
// One wave per (sequence, query head), 64 partitions per round.  Lane l
// holds 16-byte chunk l % (D / 4) of partition l / (D / 4) of each group of
// 64 / (D / 4) consecutive partitions, so one load instruction reads whole
// consecutive partials (1 KiB at D = 128); a round's partial loads are
// issued together with its log2 lse loads (lane p: partition p), so it
// costs one round trip to memory.  Each lane sums its partitions in order,
// the lane groups are then added with a fixed butterfly: the result depends
// on the partials only.
template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(DecodeArgs a) {
  constexpr int CH = D / 4;         // 16-byte chunks of a partial
  constexpr int PPI = 64 / CH;      // partitions per load instruction
  constexpr int NI = 64 / PPI;      // load instructions per 64 partitions
  const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int c = lane % CH, j = lane / CH;
  const int64_t row = (int64_t)s * a.num_q_heads + hq;
  const float* lse2 = a.ws_lse + row * a.max_parts;
  const float* po = a.ws_out + row * a.max_parts * D + 4 * c;
  // The first round's partials and sums are loaded together with the
  // length, before the partition count is known, so that the merge waits for
  // one round trip instead of two.  Slots past the count hold whatever an
  // earlier call left there; they are read (inside the workspace) but get no
  // weight and are never added.
  const int n0 = a.max_parts < 64 ? a.max_parts : 64;
  float4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (PPI * i < n0) {   // wave-uniform
      const int p = PPI * i + j < n0 ? PPI * i + j : n0 - 1;
      v[i] = *reinterpret_cast<const float4*>(po + (int64_t)p * D);
    }
  }
  float l = lane < n0 ? lse2[lane] : kNegInf;
  int len = a.seq_lens[s];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const int nparts = (len + a.partition_size - 1) / a.partition_size;
  if (nparts <= 1) return;
  float M = kNegInf, W = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int n = nparts - p0 < 64 ? nparts - p0 : 64;
    if (p0 > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (PPI * i < n) {
          const int p = PPI * i + j < n ? PPI * i + j : n - 1;
          v[i] = *reinterpret_cast<const float4*>(po + (int64_t)(p0 + p) * D);
        }
      }
      l = lse2[p0 + (lane < n ? lane : 0)];
    }
    l = lane < n ? l : kNegInf;
    float mb = l;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off));
    const float Mn = fmaxf(M, mb);
    const float alpha = M == kNegInf ? 0.f : fast_exp2(M - Mn);   // earlier rounds' sums
    M = Mn;
    W *= alpha;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] *= alpha;
    const float w = lane < n ? fast_exp2(l - M) : 0.f;
    float ws = w;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off);
    W += ws;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (PPI * i < n) {
        // the weight of the lane's partition PPI i + j (two scalar reads
        // when a load covers two partitions)
        float wi;
        if constexpr (PPI == 2) {
          const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), PPI * i));
          const float w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), PPI * i + 1));
          wi = j == 0 ? w0 : w1;
        } else {
          wi = __shfl(w, PPI * i + j);
        }
        const bool use = PPI * i + j < n;
        acc[0] = use ? fmaf(wi, v[i].x, acc[0]) : acc[0];
        acc[1] = use ? fmaf(wi, v[i].y, acc[1]) : acc[1];
        acc[2] = use ? fmaf(wi, v[i].z, acc[2]) : acc[2];
        acc[3] = use ? fmaf(wi, v[i].w, acc[3]) : acc[3];
      }
    }
  }
#pragma unroll
  for (int off = CH; off < 64; off <<= 1)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += __shfl_xor(acc[k], off);
  if (j == 0) {
    uint2 o;
    o.x = pack_bf16x2(acc[0] / W, acc[1] / W);
    o.y = pack_bf16x2(acc[2] / W, acc[3] / W);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * D + 4 * c) = o;
  }
  if (a.lse && lane == 0) a.lse[row] = (M + fast_log2(W)) * kLn2;
}

// Row layout: wave item 4 blockIdx.x + wave = (head set fastest, partition,
// sequence); waves past the last item have nothing to do.
template <int G, bool BIG, bool APP>
__global__ void __launch_bounds__(256) decode_rows_kernel(DecodeArgs a, RowsOf<APP> rows, int32_t n_items) {
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= n_items) return;
  const int hsn = a.num_kv_heads >> 2;
  const int hs = item % hsn, rest = item / hsn;
  decode_rows<G, BIG, APP, kRowBuffers<G>>(a, rows, rest % a.max_parts, hs, rest / a.max_parts);
}

// E4M3 row layout (at most 4 query heads per KV head): the same wave items.
template <int G, bool BIG>
__global__ void __launch_bounds__(256) decode_rows8_kernel(DecodeArgs a, int32_t n_items) {
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= n_items) return;
  const int hsn = a.num_kv_heads >> 2;
  const int hs = item % hsn, rest = item / hsn;
  decode_rows8<G, BIG, kRows8Buffers>(a, rest % a.max_parts, hs, rest / a.max_parts);
}

template <int G>
void launch_rows8(const DecodeArgs& a, int64_t items, hipStream_t st) {
  const dim3 grid((unsigned)((items + 3) / 4));
  if (a.log2_block_size >= 4)
    hipLaunchKernelGGL((decode_rows8_kernel<G, true>), grid, dim3(256), 0, st, a, (int32_t)items);
  else
    hipLaunchKernelGGL((decode_rows8_kernel<G, false>), grid, dim3(256), 0, st, a, (int32_t)items);
}

template <int G, bool APP>
void launch_rows(const DecodeArgs& a, const RowsOf<APP>& rows, int64_t items, hipStream_t st) {
  const dim3 grid((unsigned)((items + 3) / 4));
  if (a.log2_block_size >= 4)
    hipLaunchKernelGGL((decode_rows_kernel<G, true, APP>), grid, dim3(256), 0, st, a, rows, (int32_t)items);
  else
    hipLaunchKernelGGL((decode_rows_kernel<G, false, APP>), grid, dim3(256), 0, st, a, rows, (int32_t)items);
}

// Wave items of a row-layout launch over n sequences (-1 past int range).
int64_t row_items(const DecodeArgs& a, int32_t n) {
  const int64_t items = (int64_t)a.max_parts * (a.num_kv_heads / 4) * n;
  return items + 3 > 0x7fffffffLL ? -1 : items;
}

template <int D, int G, bool BIG, bool F8>
int launch_parts(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<D, G, BIG, F8, false>), grid, dim3(64 * kWaves<F8, G>), 0, st, a,
                     NoAppend{0});
  return (int)hipGetLastError();
}

template <int D>
int launch_merge(const DecodeArgs& a, hipStream_t st) {
  if (a.max_parts <= 1) return 0;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0, st, a);
  return (int)hipGetLastError();
}

template <int D, int G>
int launch_g(const DecodeArgs& a, hipStream_t st) {
  const bool big = a.log2_block_size >= 4;
  int e;
  if constexpr (D == 128) {
    if (a.rows) {
      const int64_t items = row_items(a, a.num_seqs);
      if (items < 0) return (int)hipErrorInvalidConfiguration;
      if (a.fp8) {
        if constexpr (G <= 4) {
          launch_rows8<G>(a, items, st);
        } else {
          return (int)hipErrorInvalidValue;   // the host sets rows with E4M3 only for G <= 4
        }
      } else {
        launch_rows<G, false>(a, NoAppend{0}, items, st);
      }
      e = (int)hipGetLastError();
      return e != 0 ? e : launch_merge<D>(a, st);
    }
  }
  if (a.fp8)
    e = big ? launch_parts<D, G, true, true>(a, st) : launch_parts<D, G, false, true>(a, st);
  else
    e = big ? launch_parts<D, G, true, false>(a, st) : launch_parts<D, G, false, false>(a, st);
  return e != 0 ? e : launch_merge<D>(a, st);
}

// Appending decode: the sequences go in launches of up to kAppendRows, each
// with its rows' slots and positions in the arguments; one merge follows.
template <int D, int G>
int launch_g_append(const DecodeArgs& a, const int64_t* slots, const int32_t* positions, hipStream_t st) {
  const bool big = a.log2_block_size >= 4;
  for (int32_t r0 = 0; r0 < a.num_seqs; r0 += kAppendRows) {
    const int32_t n = a.num_seqs - r0 < kAppendRows ? a.num_seqs - r0 : kAppendRows;
    AppendRows rows{};
    for (int32_t i = 0; i < n; ++i) {
      rows.slots[i] = slots[r0 + i];
      rows.pos[i] = positions[r0 + i];
    }
    // rows r0 .. r0 + n - 1 are rows 0 .. n - 1 of this launch
    DecodeArgs b = a;
    const int64_t hq = a.num_q_heads;
    b.num_seqs = n;
    b.out = static_cast<uint16_t*>(a.out) + r0 * hq * D;
    if (a.lse) b.lse = a.lse + r0 * hq;
    b.q = static_cast<const uint16_t*>(a.q) + r0 * hq * D;
    b.block_tables = a.block_tables + (int64_t)r0 * a.bt_stride;
    b.seq_lens = a.seq_lens + r0;
    if (a.ws_out) {
      b.ws_out = a.ws_out + r0 * hq * a.max_parts * D;
      b.ws_lse = a.ws_lse + r0 * hq * a.max_parts;
    }
    b.new_key = static_cast<const uint16_t*>(a.new_key) + r0 * a.new_key_stride;
    b.new_value = static_cast<const uint16_t*>(a.new_value) + r0 * a.new_value_stride;
    b.wr_tables = a.wr_tables + (int64_t)r0 * a.bt_stride;
    b.wr_lens = a.wr_lens + r0;
    if constexpr (D == 128) {
      if (a.rows) {
        const int64_t items = row_items(a, n);
        if (items < 0) return (int)hipErrorInvalidConfiguration;
        launch_rows<G, true>(b, rows, items, st);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
        continue;
      }
    }
    const dim3 grid(a.max_parts, a.num_kv_heads, n);
    if (big)
      hipLaunchKernelGGL((decode_partition_kernel<D, G, true, false, true>), grid, dim3(64 * kWaves<false, G>), 0, st, b,
                         rows);
    else
      hipLaunchKernelGGL((decode_partition_kernel<D, G, false, false, true>), grid, dim3(64 * kWaves<false, G>), 0, st, b,
                         rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return launch_merge<D>(a, st);
}

template <int D>
int launch_d(const DecodeArgs& a, hipStream_t st) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<D, 1>(a, st);
    case 2: return launch_g<D, 2>(a, st);
    case 3: return launch_g<D, 3>(a, st);
    case 4: return launch_g<D, 4>(a, st);
    case 5: return launch_g<D, 5>(a, st);
    case 6: return launch_g<D, 6>(a, st);
    case 7: return launch_g<D, 7>(a, st);
    case 8: return launch_g<D, 8>(a, st);
  }
  return (int)hipErrorInvalidValue;
}

template <int D>
int launch_d_append(const DecodeArgs& a, const int64_t* slots, const int32_t* positions, hipStream_t st) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g_append<D, 1>(a, slots, positions, st);
    case 2: return launch_g_append<D, 2>(a, slots, positions, st);
    case 3: return launch_g_append<D, 3>(a, slots, positions, st);
    case 4: return launch_g_append<D, 4>(a, slots, positions, st);
    case 5: return launch_g_append<D, 5>(a, slots, positions, st);
    case 6: return launch_g_append<D, 6>(a, slots, positions, st);
    case 7: return launch_g_append<D, 7>(a, slots, positions, st);
    case 8: return launch_g_append<D, 8>(a, slots, positions, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

// Split-K scratch of the allocation-free decode entry point: a file-scope
// device array (each GPU the library runs on holds its own copy until the
// process ends).  In host code `scratch` only stands for the symbol; its
// device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

int static_decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return 0;
}

int launch_decode_merge(const DecodeArgs& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_merge<64>(a, st) : launch_merge<128>(a, st);
}

int launch_paged_decode(const DecodeArgs& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

int launch_paged_decode_append(const DecodeArgs& a, const int64_t* slots, const int32_t* positions, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_d_append<64>(a, slots, positions, st)
                          : launch_d_append<128>(a, slots, positions, st);
}

}  // namespace pa
