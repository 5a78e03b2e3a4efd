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
//   * K and V are stored row-major [key][d]; the V^T operand is read with
//     gfx950's transposing LDS read (ds_read_b64_tr_b16).  Loads of keys past
//     the sequence end are redirected to a written row and those keys are
//     masked out of the softmax, so bytes of unwritten slots (NaN, say) can
//     never reach a product.
//   * With B >= 16 each wave stages one 16-key run of a block per tile: the
//     block id is a scalar load and the row base a scalar address.
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
//     computed (register staging, double-buffered LDS, one barrier per tile);
//     block-table entries are fetched one further tile ahead.
#include "../internal.hpp"
#include "common.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// Staged K/V pieces use a native vector type: copies of it are plain loads
// and stores, which keeps the staging arrays in registers.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKeys = 64;        // keys per tile
constexpr int kQB = 1;           // 32-query blocks per wave (two: 10 % slower, see below)
constexpr int kQ = 32 * kQB;     // queries per wave
constexpr int kXcds = 8;         // accelerator dies of an MI355X, one L2 each
constexpr int kSortMax = 256;    // requests ordered by work up to this many
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kSlack = 8.0f;

// Both tiles are row-major [key][d] in LDS of 64 four-byte banks.  K rows
// are padded to D + 8 elements (the rows read by one S^T operand fall on
// distinct banks).  V rows are padded to D + 32 elements, a stride of 16 (or
// 48) banks: a transposing read serves 32 lanes at a time, two 16-lane groups
// 16 elements apart, each reading 8 bytes from four consecutive rows, and with
// this stride the 32 lanes cover all 64 banks once (with D + 16 they met
// twice on half the banks; measured as 25 % of LDS cycles lost to conflicts).
template <int D>
struct Smem {
  static constexpr int kRow = D + 8;
  static constexpr int kVRow = D + 32;
  uint16_t k[2][kKeys * kRow];
  uint16_t v[2][kKeys * kVRow];
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte rows addressed by lanes a, a + 4, a + 8, a + 12.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

template <int D, int HW, bool CAUSAL, bool BIG, bool F8>
__global__ void __launch_bounds__(256) prefill_kernel(PrefillArgs a) {
  constexpr int QS = 4 / HW;                 // 32-query sub-tiles per work-group
  constexpr int DS = D / 16;                 // MFMA k-steps over head_dim
  constexpr int DB = D / 32;                 // 32-row blocks of head_dim in O^T
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int UPT = 32 * CPR / 256;        // (key pair, chunk) units per thread
  // E4M3 caches (F8): a row is D bytes, in 16-byte chunks of 16 codes that
  // become two 16-byte bf16 pieces in LDS
  constexpr int CPR8 = D / 16;               // chunks per row
  constexpr int KPI8 = 64 / CPR8;            // BIG: keys per load instruction
  constexpr int NU8 = 64 * CPR8 / 256;       // otherwise: (key, chunk) units per thread
  __shared__ Smem<D> sm;

  // Work-groups are dealt to the 8 XCDs round-robin by linear id, and each
  // XCD has its own L2.  Work item (request i, head group y, query tile) is
  // placed so that all query tiles of one (i, y) land on the same XCD, one
  // after another: they walk the same K/V tiles at about the same time, so
  // the XCD's L2 serves those tiles to all of them.  Group n = i * Y + y goes
  // to XCD n % 8; with 8 head groups each XCD owns one KV head.
  const int X = (a.max_query_len + kQ * QS - 1) / (kQ * QS);   // query tiles per request
  const int Y = a.num_q_heads / HW;                             // head groups
  const int xcd = blockIdx.x & (kXcds - 1), k_in_xcd = blockIdx.x / kXcds;
  const int grp = xcd + kXcds * (k_in_xcd / X);
  if (grp >= a.num_seqs * Y) return;
  const int y = grp % Y;                      // head group
  const int xt = k_in_xcd % X;                // 0 = the request's last (heaviest) query tile
  const int tid = threadIdx.x, lane = tid & 63;

  // Requests are taken in order of decreasing work, q_len (2 kv_len - q_len)
  // (twice the visible query-key pairs), ties in index order, so that the
  // longest start first and the work-groups of an XCD finish together.  The
  // rank is found by counting; with more than kSortMax requests the index
  // order is kept.
  int i = grp / Y;
  if (a.num_seqs > 1 && a.num_seqs <= kSortMax) {
    __shared__ int64_t s_cost[kSortMax];
    __shared__ int s_req;
    for (int c = tid; c < a.num_seqs; c += 256) {
      const int ql = a.query_start_loc[c + 1] - a.query_start_loc[c];
      int kv = a.seq_lens[c];
      kv = kv > a.max_seq_len ? a.max_seq_len : kv;
      s_cost[c] = ql > 0 && kv >= ql ? (int64_t)ql * (2 * (int64_t)kv - ql) : 0;
    }
    __syncthreads();
    const int rank = i;
    for (int c = tid; c < a.num_seqs; c += 256) {
      const int64_t mine = s_cost[c];
      int r = 0;
      for (int j = 0; j < a.num_seqs; ++j) {
        const int64_t o = s_cost[j];
        r += (o > mine) | ((o == mine) & (j < c));
      }
      if (r == rank) s_req = c;
    }
    __syncthreads();
    i = s_req;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, col = lane & 31;

  const int q_begin = a.query_start_loc[i];
  const int q_len = a.query_start_loc[i + 1] - q_begin;
  int kv_len = a.seq_lens[i];
  kv_len = kv_len > a.max_seq_len ? a.max_seq_len : kv_len;
  const int ctx = kv_len - q_len;            // absolute position of query 0
  const int span = kQ * QS;
  const int q0 = (X - 1 - xt) * span;                    // heaviest tiles first
  if (q_len <= 0 || q0 >= q_len || ctx < 0) return;

  const int G = a.num_q_heads / a.num_kv_heads;
  const int h = y * HW + wave % HW;                      // this wave's query head
  const int g = (y * HW) / G;                            // shared KV head
  const int qw = q0 + (wave / HW) * kQ;                  // this wave's first query
  const int lgB = a.log2_block_size;
  const int Bmask = (1 << lgB) - 1;
  const int64_t row_elems = (int64_t)a.num_kv_heads * D;
  const int64_t bstride = a.cache_block_stride;
  const uint16_t* kc = static_cast<const uint16_t*>(a.key_cache) + (int64_t)g * D;
  const uint16_t* vc = static_cast<const uint16_t*>(a.value_cache) + (int64_t)g * D;
  const int32_t* bt_row = a.block_tables + (int64_t)i * a.bt_stride;
  // A negative scale is applied as |scale| on -q (flipping q's sign bits is
  // exact), so the running maximum can always be taken on raw scores.
  const float scale = fabsf(a.scale) * kLog2e;
  const uint32_t qflip = a.scale < 0.f ? 0x80008000u : 0u;

  // keys this work-group needs: causal -> up to the position of its last query
  const int q_last = (q0 + span < q_len ? q0 + span : q_len) - 1;
  const int kv_end = CAUSAL ? ctx + q_last + 1 : kv_len;
  const int n_tiles = (kv_end + kKeys - 1) / kKeys;

  // Q^T operands: in query block qb the lane holds query qw + 32 qb + col,
  // d = 16 ks + 8 hf .. +8.
  uint4 qreg[kQB][DS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    int qi = qw + 32 * qb + col;
    qi = qi < q_len ? qi : q_len - 1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)(q_begin + qi) * a.num_q_heads + h) * D;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 16 * ks + 8 * hf);
      qreg[qb][ks] = make_uint4(v.x ^ qflip, v.y ^ qflip, v.z ^ qflip, v.w ^ qflip);
    }
  }

  // Tile staging.  Keys at or past kv_end are loaded from a valid row
  // instead (the wave's first key of the tile, or key 0) and are removed from the
  // softmax by the score mask below, so whatever bytes unwritten slots hold
  // never reach a product and the loads need no branch.
  //   BIG (B >= 16): wave w stages keys n0 + 16 w .. n0 + 16 w + 15, which lie
  //   in one block; the block id is a scalar load and the row base a scalar
  //   address, each lane adds a fixed 32-bit offset.
  //   otherwise: unit u = (key pair kp, 16-byte chunk c); every key looks up
  //   its own block.
  constexpr int KPI = 64 / CPR;              // BIG: keys per load instruction
  constexpr int NI = BIG ? 16 / KPI : 2 * UPT;
  const int kr0 = lane / CPR, chunk = lane % CPR;
  uint32_t voff[BIG ? NI : 1];
  if constexpr (BIG) {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      voff[j] = (uint32_t)(((KPI * j + kr0) * row_elems + (int64_t)g * D + 8 * chunk) * 2);
  }
  const uint32_t voff_row0 = (uint32_t)(((int64_t)g * D + 8 * chunk) * 2);
  int kp_[UPT], ch_[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid + 256 * u;
    kp_[u] = unit / CPR;
    ch_[u] = unit % CPR;
  }
  int blk_next[BIG ? 1 : UPT][2];             // table entries, one tile ahead of the loads
  constexpr int NS = F8 ? (BIG ? 16 / KPI8 : NU8) : NI;
  u32x4_t kr[NS], vr[NS];                     // staged K/V of the tile being loaded
  // F8 staging: lane -> (key kr08 of each load, chunk chunk8); byte offsets
  const int kr08 = lane / CPR8, chunk8 = lane % CPR8;
  uint32_t voff8[F8 && BIG ? NS : 1];
  if constexpr (F8 && BIG) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      voff8[j] = (uint32_t)((KPI8 * j + kr08) * row_elems + (int64_t)g * D + 16 * chunk8);
  }
  const uint32_t voff8_row0 = (uint32_t)((int64_t)g * D + 16 * chunk8);
  int key8_[F8 && !BIG ? NU8 : 1], ch8_[F8 && !BIG ? NU8 : 1], blk8_[F8 && !BIG ? NU8 : 1];
  if constexpr (F8 && !BIG) {
#pragma unroll
    for (int u = 0; u < NU8; ++u) {
      key8_[u] = (tid + 256 * u) / CPR8;
      ch8_[u] = (tid + 256 * u) % CPR8;
    }
  }

  auto wave_key = [&](int tile) {
    const int kw = tile * kKeys + 16 * wave;
    return kw < kv_end ? kw : 0;
  };
  auto fetch_table = [&](int tile) {
    if constexpr (F8 && !BIG) {
#pragma unroll
      for (int u = 0; u < NU8; ++u) {
        int p = tile * kKeys + key8_[u];
        p = p < kv_end ? p : 0;
        const int b = bt_row[p >> lgB];
        blk8_[u] = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
      }
    } else if constexpr (BIG) {
      int b = bt_row[wave_key(tile) >> lgB];
      b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
      blk_next[0][0] = __builtin_amdgcn_readfirstlane(b);
    } else {
#pragma unroll
      for (int u = 0; u < UPT; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          int p = tile * kKeys + 2 * kp_[u] + e;
          p = p < kv_end ? p : 0;
          int b = bt_row[p >> lgB];
          blk_next[u][e] = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
        }
    }
  };
  auto issue_loads = [&](int tile) {
    if constexpr (F8 && BIG) {
      const int kw = wave_key(tile);
      const int lim = kv_end - 1 - kw;        // rows 0 .. lim of the wave's 16 are keys
      const int64_t base = (int64_t)blk_next[0][0] * bstride + (int64_t)(kw & Bmask) * row_elems;
      const char* kb = reinterpret_cast<const char*>(a.key_cache) + base;
      const char* vb = reinterpret_cast<const char*>(a.value_cache) + base;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const uint32_t off = KPI8 * j + kr08 <= lim ? voff8[j] : voff8_row0;
        kr[j] = *reinterpret_cast<const u32x4_t*>(kb + off);
        vr[j] = *reinterpret_cast<const u32x4_t*>(vb + off);
      }
    } else if constexpr (F8) {
#pragma unroll
      for (int u = 0; u < NU8; ++u) {
        int p = tile * kKeys + key8_[u];
        p = p < kv_end ? p : 0;
        const int64_t off = (int64_t)blk8_[u] * bstride + (int64_t)(p & Bmask) * row_elems + (int64_t)g * D +
                            16 * ch8_[u];
        kr[u] = *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(a.key_cache) + off);
        vr[u] = *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(a.value_cache) + off);
      }
    } else if constexpr (BIG) {
      const int kw = wave_key(tile);
      const int lim = kv_end - 1 - kw;        // rows 0 .. lim of the wave's 16 are keys
      const int64_t base = ((int64_t)blk_next[0][0] * bstride + (int64_t)(kw & Bmask) * row_elems) * 2;
      const char* kb = reinterpret_cast<const char*>(a.key_cache) + base;
      const char* vb = reinterpret_cast<const char*>(a.value_cache) + base;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint32_t off = KPI * j + kr0 <= lim ? voff[j] : voff_row0;
        kr[j] = *reinterpret_cast<const u32x4_t*>(kb + off);
        vr[j] = *reinterpret_cast<const u32x4_t*>(vb + off);
      }
    } else {
#pragma unroll
      for (int u = 0; u < UPT; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          int p = tile * kKeys + 2 * kp_[u] + e;
          p = p < kv_end ? p : 0;
          const int64_t off = (int64_t)blk_next[u][e] * bstride + (int64_t)(p & Bmask) * row_elems + 8 * ch_[u];
          kr[2 * u + e] = *reinterpret_cast<const u32x4_t*>(kc + off);
          vr[2 * u + e] = *reinterpret_cast<const u32x4_t*>(vc + off);
        }
    }
  };
  // 16 E4M3 codes -> two 16-byte pieces of bf16 (exact conversion)
  auto store8 = [&](uint16_t* dst, const u32x4_t c) __attribute__((always_inline)) {
    u32x4_t lo, hi;
    lo[0] = e4m3x2_to_bf16x2<false>(c[0]);
    lo[1] = e4m3x2_to_bf16x2<true>(c[0]);
    lo[2] = e4m3x2_to_bf16x2<false>(c[1]);
    lo[3] = e4m3x2_to_bf16x2<true>(c[1]);
    hi[0] = e4m3x2_to_bf16x2<false>(c[2]);
    hi[1] = e4m3x2_to_bf16x2<true>(c[2]);
    hi[2] = e4m3x2_to_bf16x2<false>(c[3]);
    hi[3] = e4m3x2_to_bf16x2<true>(c[3]);
    *reinterpret_cast<u32x4_t*>(dst) = lo;
    *reinterpret_cast<u32x4_t*>(dst + 8) = hi;
  };
  auto store_tile = [&](int buf) {
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int key = BIG ? 16 * wave + KPI8 * j + kr08 : key8_[BIG ? 0 : j];
        const int c = BIG ? chunk8 : ch8_[BIG ? 0 : j];
        store8(&sm.k[buf][key * Smem<D>::kRow + 16 * c], kr[j]);
        store8(&sm.v[buf][key * Smem<D>::kVRow + 16 * c], vr[j]);
      }
    } else if constexpr (BIG) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int key = 16 * wave + KPI * j + kr0;
        *reinterpret_cast<u32x4_t*>(&sm.k[buf][key * Smem<D>::kRow + 8 * chunk]) = kr[j];
        *reinterpret_cast<u32x4_t*>(&sm.v[buf][key * Smem<D>::kVRow + 8 * chunk]) = vr[j];
      }
    } else {
#pragma unroll
      for (int u = 0; u < UPT; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int key = 2 * kp_[u] + e;
          *reinterpret_cast<u32x4_t*>(&sm.k[buf][key * Smem<D>::kRow + 8 * ch_[u]]) = kr[2 * u + e];
          *reinterpret_cast<u32x4_t*>(&sm.v[buf][key * Smem<D>::kVRow + 8 * ch_[u]]) = vr[2 * u + e];
        }
    }
  };

  f32x16_t o[kQB][DB];
  float m[kQB], l[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][b][r] = 0.f;
    m[qb] = kNegInf;
    l[qb] = 0.f;
  }

  // Staging is unconditional: tiles past the end read valid rows, so no
  // branch separates a load from its use.
  fetch_table(0);
  issue_loads(0);
  fetch_table(1);
  store_tile(0);
  issue_loads(1);
  fetch_table(2);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const uint16_t* K = sm.k[buf];
    const uint16_t* V = sm.v[buf];
    // S^T[key][query] for the two 32-key halves of the tile and each query
    // block.  The accumulations are independent: their MFMAs alternate, every
    // K operand read from LDS feeds all query blocks, and the next k-step's K
    // operands are read before this step's MFMAs issue.
    f32x16_t s[kQB][2];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
    {
      const uint16_t* krow0 = &K[col * Smem<D>::kRow + 8 * hf];
      const uint16_t* krow1 = &K[(32 + col) * Smem<D>::kRow + 8 * hf];
      uint4 ka0 = *reinterpret_cast<const uint4*>(krow0);
      uint4 ka1 = *reinterpret_cast<const uint4*>(krow1);
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) {
        uint4 kn0 = ka0, kn1 = ka1;
        if (ks + 1 < DS) {
          kn0 = *reinterpret_cast<const uint4*>(krow0 + 16 * (ks + 1));
          kn1 = *reinterpret_cast<const uint4*>(krow1 + 16 * (ks + 1));
        }
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          s[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka0), as_bf16x8(qreg[qb][ks]), s[qb][0], 0, 0, 0);
          s[qb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka1), as_bf16x8(qreg[qb][ks]), s[qb][1], 0, 0, 0);
        }
        ka0 = kn0;
        ka1 = kn1;
      }
    }
    // mask and tile max on raw scores.  Register r of half kb holds key
    // n0 + 32 kb + 8 (r / 4) + 4 hf + r % 4; a key is visible iff its offset
    // 32 kb + 8 (r / 4) + r % 4 is at most `lim` (one compare per score, on
    // tiles that reach past the query block's first query only).
    const int n0 = t * kKeys;
    uint32_t pb[kQB][2][2][4];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int qpos = ctx + qw + 32 * qb + col;     // absolute position of the lane's query
      const int lim = (CAUSAL ? qpos : kv_len - 1) - n0 - 4 * hf;
      const bool need_mask = n0 + kKeys - 1 > (CAUSAL ? ctx + qw + 32 * qb : kv_len - 1);
      float mt = kNegInf;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[qb][kb][r] = 32 * kb + 8 * (r >> 2) + (r & 3) <= lim ? s[qb][kb][r] : kNegInf;
            mt = fmaxf(mt, s[qb][kb][r]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[qb][kb][r]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale;
      if (mt > m[qb] + kSlack) {
        const float alpha = fast_exp2(m[qb] - mt);
        l[qb] *= alpha;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qb][b][r] *= alpha;
        m[qb] = mt;
      }
      // P^T in bf16: B operand slots s of lane half hf <-> registers 8 ks + s;
      // weights are exp2(score * scale - m), and their bf16 values are summed.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float e0 = fast_exp2(fmaf(s[qb][kb][8 * ks + 2 * w], scale, -m[qb]));
            const float e1 = fast_exp2(fmaf(s[qb][kb][8 * ks + 2 * w + 1], scale, -m[qb]));
            const uint32_t pk = pack_bf16x2(e0, e1);
            pb[qb][kb][ks][w] = pk;
            l[qb] = dot2_bf16(pk, 0x3F803F80u, l[qb]);
          }
    }
    // O^T[d][query] += V^T[d][key] P^T[key][query]; slot s of lane half hf in
    // step (kb, ks) is key 32 kb + 16 ks + 8 (s / 4) + 4 hf + s % 4.  The V^T
    // operand (lane: d = 32 b + col) comes from row-major V with transposing
    // reads: in each 16-lane group (d = dg .. dg + 15), lane a + 4 c points at
    // V[key0 + c][dg + 4 a], which hands lane j the 4 keys of d = dg + j.
    const int tr_a = lane & 3, tr_c = (lane >> 2) & 3, tr_g = (lane >> 4) & 1;
    const uint16_t* vbase = &V[tr_c * Smem<D>::kVRow + 16 * tr_g + 4 * tr_a + 4 * hf * Smem<D>::kVRow];
    auto read_vt = [&](int step, int b) {
      const int kb = step >> 1, ks = step & 1;
      const uint16_t* src = vbase + (32 * kb + 16 * ks) * Smem<D>::kVRow + 32 * b;
      const uint2 lo = lds_read_tr16(src);
      const uint2 hi = lds_read_tr16(src + 8 * Smem<D>::kVRow);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    uint4 va[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) va[b] = read_vt(0, b);
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const int kb = step >> 1, ks = step & 1;
      uint4 pv[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        pv[qb] = make_uint4(pb[qb][kb][ks][0], pb[qb][kb][ks][1], pb[qb][kb][ks][2], pb[qb][kb][ks][3]);
      uint4 vn[DB];
#pragma unroll
      for (int b = 0; b < DB; ++b) vn[b] = step + 1 < 4 ? read_vt(step + 1, b) : va[b];
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          o[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[b]), as_bf16x8(pv[qb]), o[qb][b], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < DB; ++b) va[b] = vn[b];
    }
    // stage the next tile into the other buffer and start the one after
    store_tile(buf ^ 1);
    issue_loads(t + 2);
    fetch_table(t + 3);
    __syncthreads();
  }

  // normalise and write: in query block qb the lane owns query
  // qw + 32 qb + col, d = 32 b + 8 (r / 4) + 4 hf + r % 4
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const int qi = qw + 32 * qb + col;
    if (qi < q_len) {
      const float inv = lt > 0.f ? (F8 ? a.v_scale / lt : 1.f / lt) : 0.f;
      uint16_t* op = static_cast<uint16_t*>(a.out) + ((int64_t)(q_begin + qi) * a.num_q_heads + h) * D;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t lo = pack_bf16x2(o[qb][b][4 * rr] * inv, o[qb][b][4 * rr + 1] * inv);
          const uint32_t hi = pack_bf16x2(o[qb][b][4 * rr + 2] * inv, o[qb][b][4 * rr + 3] * inv);
          *reinterpret_cast<uint2*>(op + 32 * b + 8 * rr + 4 * hf) = make_uint2(lo, hi);
        }
    }
  }
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
      hipLaunchKernelGGL((prefill_kernel<D, HW, true, true, true>), grid, dim3(256), 0, st, a);
    else if (a.causal)
      hipLaunchKernelGGL((prefill_kernel<D, HW, true, false, true>), grid, dim3(256), 0, st, a);
    else if (big)
      hipLaunchKernelGGL((prefill_kernel<D, HW, false, true, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_kernel<D, HW, false, false, true>), grid, dim3(256), 0, st, a);
  } else if (a.causal && big)
    hipLaunchKernelGGL((prefill_kernel<D, HW, true, true, false>), grid, dim3(256), 0, st, a);
  else if (a.causal)
    hipLaunchKernelGGL((prefill_kernel<D, HW, true, false, false>), grid, dim3(256), 0, st, a);
  else if (big)
    hipLaunchKernelGGL((prefill_kernel<D, HW, false, true, false>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, HW, false, false, false>), grid, dim3(256), 0, st, a);
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

int launch_paged_prefill(const PrefillArgs& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace pa
