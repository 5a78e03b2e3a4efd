// Chunked-prefill attention body for gfx950 MFMA, shared by the prefill
// kernel and the mixed-batch kernel (see paged_prefill.hip for the design).
#pragma once

#include <type_traits>

#include "../internal.hpp"
#include "common.hpp"

namespace pa {
namespace prefill_body {

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

// LDS tiles (K and V alike): 64 rows [key][d] of D bf16 elements, no
// padding.  Chunk c (elements 8c .. 8c + 7) of row r is stored at chunk
// position c ^ chunk_swz(r).  LDS has 64 four-byte banks.  With D = 128 a
// row spans all of them and the XOR takes the row's low four bits with its
// two halves exchanged; with D = 64 two rows share the banks and the XOR
// takes row bits 1..3, bit 1 moved to the top.  Either way:
//   * the S^T operand read (16 lanes, rows r .. r + 15, one chunk each)
//     meets 16 different chunk positions (D = 64: 8 per row parity);
//   * a transposing V^T read (32 lanes, 4 consecutive rows from a multiple
//     of 4, 4 consecutive chunks from a multiple of 4, 8 bytes per lane)
//     puts the 4 rows into 4 different 64-byte groups of banks.
template <int D>
__device__ __forceinline__ int chunk_swz(int row) {
  return D == 128 ? ((row & 3) << 2) | ((row >> 2) & 3) : (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}
// element offset of chunk c of row r in a tile
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * D + 8 * (chunk ^ chunk_swz<D>(row));
}

// One 16-byte piece per lane from global memory straight into LDS: lane l
// writes dst + 16 l (dst is the same for the whole wave).
__device__ __forceinline__ void load_to_lds16(const void* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte rows addressed by lanes a, a + 4, a + 8, a + 12.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// The prefill work of work-group number bid (every work-group runs it with
// 256 threads, two work-groups per CU).
// KO, the form of the per-key byte offsets with block size < 16: 0 64-bit,
// 1 32-bit (every byte offset of a cache fits), 2 32-bit with block size 1
// (a key's offset is its block's alone).
template <int D, int HW, bool CAUSAL, bool BIG, bool F8, int KO>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, const int bid) {
  constexpr int QS = 4 / HW;                 // 32-query sub-tiles per work-group
  constexpr int DS = D / 16;                 // MFMA k-steps over head_dim
  constexpr int DB = D / 32;                 // 32-row blocks of head_dim in O^T
  constexpr int CPR = D / 8;                 // 16-byte bf16 chunks per K/V row
  // E4M3 caches (F8): a row is D bytes, in 16-byte chunks of 16 codes that
  // become two bf16 chunks in LDS
  constexpr int CPR8 = D / 16;               // chunks per row
  constexpr int KPI8 = 64 / CPR8;            // keys per load instruction
  // two buffers of each tile, as separate objects: the compiler then sees
  // that reads of one never wait for the LDS writes in flight to the other
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[kKeys * D], s_k1[kKeys * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v0[kKeys * D], s_v1[kKeys * D];

  // Work-groups are dealt to the 8 XCDs round-robin by linear id, and each
  // XCD has its own L2.  Work item (request i, head group y, query tile) is
  // placed so that all query tiles of one (i, y) land on the same XCD, one
  // after another: they walk the same K/V tiles at about the same time, so
  // the XCD's L2 serves those tiles to all of them.  Group n = i * Y + y goes
  // to XCD n % 8; with 8 head groups each XCD owns one KV head.
  const int X = (a.max_query_len + kQ * QS - 1) / (kQ * QS);   // query tiles per request
  const int Y = a.num_q_heads / HW;                             // head groups
  const int xcd = bid & (kXcds - 1), k_in_xcd = bid / kXcds;
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

  // Tile staging.  Wave w stages keys n0 + 16 w .. n0 + 16 w + 15 of tile
  // n0 / 64, KPI of them per load instruction (bf16: 64 / CPR; E4M3: KPI8),
  // the lane taking key kr0 and one chunk.  Keys at or past kv_end are loaded
  // from a valid row instead (the wave's first key of the tile, or key 0) and
  // are removed from the softmax by the score mask below, so whatever bytes
  // unwritten slots hold never reach a product and the loads need no branch.
  //   BIG (B >= 16): the 16 keys lie in one block; its id is a scalar load
  //   and the row base a scalar address, each lane adds a fixed offset.
  //   otherwise: every key looks up its own block.
  // bf16: the lane at byte 16 l of an instruction's LDS window holds row
  // KPI j + l / CPR, chunk position l % CPR, i.e. chunk cg[j] of that row.
  constexpr int KPI = F8 ? KPI8 : 64 / CPR;
  constexpr int NI = 16 / KPI;               // load instructions per wave and tile, each of K and V
  const int kr0 = lane / (F8 ? CPR8 : CPR);
  const int pos = lane % (F8 ? CPR8 : CPR);  // bf16: chunk position; E4M3: code chunk
  uint32_t voff[NI], voff0[NI];              // byte offsets of the lane's row and of row 0 (BIG)
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int cg = F8 ? pos : pos ^ chunk_swz<D>(KPI * j + kr0);
    const int64_t cb = (int64_t)g * D * (F8 ? 1 : 2) + 16 * cg;
    voff[j] = (uint32_t)((KPI * j + kr0) * row_elems * (F8 ? 1 : 2) + cb);
    voff0[j] = (uint32_t)cb;
  }
  u32x4_t kr[F8 ? NI : 1], vr[F8 ? NI : 1];  // E4M3: staged codes of the tile being loaded

  auto wave_key = [&](int tile) {
    const int kw = tile * kKeys + 16 * wave;
    return kw < kv_end ? kw : 0;
  };
  auto clamp_blk = [&](int b) { return b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b); };
  // Block ids.  BIG: a wave needs one table entry per tile; lane i of `tab`
  // holds the entry of tile win + i (a window of 64 tiles, read with
  // readlane), and `tab_next` the following window, fetched one window
  // ahead, so the tile loop itself issues no table loads.  Otherwise: the
  // entries of each lane's NI keys, fetched two tiles ahead (before the
  // loads of the next tile) and clamped where they are used.
  int tab = 0, tab_next = 0, win = 0;
  auto load_window = [&](int w0) {
    return bt_row[wave_key(w0 + lane) >> lgB];
  };
  int ent[BIG ? 1 : NI], ent_next[BIG ? 1 : NI];
  auto fetch_entries = [&](int tile, int (&e)[BIG ? 1 : NI]) {
    if constexpr (!BIG) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        int p = tile * kKeys + 16 * wave + KPI * j + kr0;
        p = p < kv_end ? p : 0;
        e[j] = bt_row[KO == 2 ? p : p >> lgB];
      }
    }
  };
  // the window must cover `tile` (called with tiles in increasing order, one
  // window at a time)
  auto advance_window = [&](int tile) {
    if constexpr (BIG) {
      if (tile >= win + 64) {
        win += 64;
        tab = tab_next;
        if (win + 64 < n_tiles) tab_next = load_window(win + 64);
      }
    }
  };
  // B >= 16: a wave's 16 rows of a tile lie in one block, so their base is
  // wave-uniform (a scalar address) and each lane adds a 32-bit offset;
  // rows past `lim` (keys at or past kv_end) load the wave's first row.
  struct Rows {
    int64_t base;   // bytes from the cache's start
    int lim;        // rows 0 .. lim of the wave's 16 are keys
  };
  auto tile_rows = [&](int tile) __attribute__((always_inline)) {
    const int kw = wave_key(tile);
    const int blk = clamp_blk(__builtin_amdgcn_readlane(tab, tile - win));
    return Rows{((int64_t)blk * bstride + (int64_t)(kw & Bmask) * row_elems) * (F8 ? 1 : 2), kv_end - 1 - kw};
  };
  // (the empty asm keeps the offset a 32-bit register value, so that the
  // address stays scalar base + lane offset instead of becoming a select
  // between two 64-bit addresses)
  auto row_off = [&](const Rows& r, int j, auto wholec) __attribute__((always_inline)) {
    uint32_t off = decltype(wholec)::value || KPI * j + kr0 <= r.lim ? voff[j] : voff0[j];
    asm("" : "+v"(off));
    return off;
  };
  // B < 16: byte offset of the piece that load j of `tile` fetches (every
  // key looks up its own block)
  auto key_off = [&](int tile, int j) __attribute__((always_inline)) {
    int p = tile * kKeys + 16 * wave + KPI * j + kr0;
    p = p < kv_end ? p : 0;
    if constexpr (KO == 2) {
      // block size 1: the key is row 0 of its block (32-bit offsets, as KO 1)
      uint32_t off = (uint32_t)clamp_blk(ent[j]) * (uint32_t)(bstride * (F8 ? 1 : 2)) + voff0[j];
      asm("" : "+v"(off));
      return off;
    } else if constexpr (KO == 1) {
      // every byte offset of the cache fits in 32 bits (checked on the host)
      uint32_t off = (uint32_t)clamp_blk(ent[j]) * (uint32_t)(bstride * (F8 ? 1 : 2)) +
                     (uint32_t)(p & Bmask) * (uint32_t)(row_elems * (F8 ? 1 : 2)) + voff0[j];
      asm("" : "+v"(off));
      return off;
    } else {
      return ((int64_t)clamp_blk(ent[j]) * bstride + (int64_t)(p & Bmask) * row_elems) * (F8 ? 1 : 2) + voff0[j];
    }
  };
  using KeyOff = decltype(key_off(0, 0));
  const char* kcb = static_cast<const char*>(a.key_cache);
  const char* vcb = static_cast<const char*>(a.value_cache);
  // bf16, B >= 16: the wave's rows of one tile of `cache` into LDS tile dst
  // (WHOLE asserts that all 16 rows are keys)
  auto load_rows = [&](const char* cache, const Rows r, uint16_t* dst, auto wholec) __attribute__((always_inline)) {
    const char* base = cache + r.base;
#pragma unroll
    for (int j = 0; j < NI; ++j) load_to_lds16(base + row_off(r, j, wholec), dst + (16 * wave + KPI * j) * D);
  };
  // bf16: tile `tile` into LDS tiles kd / vd (rows 16 w .. 16 w + 15)
  auto load_tile = [&](int tile, uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
    if constexpr (BIG) {
      const Rows r = tile_rows(tile);
      load_rows(kcb, r, kd, std::false_type());
      load_rows(vcb, r, vd, std::false_type());
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const KeyOff off = key_off(tile, j);
        load_to_lds16(kcb + off, kd + (16 * wave + KPI * j) * D);
        load_to_lds16(vcb + off, vd + (16 * wave + KPI * j) * D);
      }
    }
  };
  // E4M3: codes of tile `tile` into registers
  auto issue_loads = [&](int tile) __attribute__((always_inline)) {
    if constexpr (BIG) {
      const Rows r = tile_rows(tile);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint32_t off = row_off(r, j, std::false_type());
        kr[j] = *reinterpret_cast<const u32x4_t*>(kcb + r.base + off);
        vr[j] = *reinterpret_cast<const u32x4_t*>(vcb + r.base + off);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const KeyOff off = key_off(tile, j);
        kr[j] = *reinterpret_cast<const u32x4_t*>(kcb + off);
        vr[j] = *reinterpret_cast<const u32x4_t*>(vcb + off);
      }
    }
  };
  // 16 E4M3 codes (code chunk c of row `key`) -> bf16 chunks 2c and 2c + 1
  // (exact conversion)
  auto store8 = [&](uint16_t* tile, int key, int c, const u32x4_t x) __attribute__((always_inline)) {
    u32x4_t lo, hi;
    lo[0] = e4m3x2_to_bf16x2<false>(x[0]);
    lo[1] = e4m3x2_to_bf16x2<true>(x[0]);
    lo[2] = e4m3x2_to_bf16x2<false>(x[1]);
    lo[3] = e4m3x2_to_bf16x2<true>(x[1]);
    hi[0] = e4m3x2_to_bf16x2<false>(x[2]);
    hi[1] = e4m3x2_to_bf16x2<true>(x[2]);
    hi[2] = e4m3x2_to_bf16x2<false>(x[3]);
    hi[3] = e4m3x2_to_bf16x2<true>(x[3]);
    *reinterpret_cast<u32x4_t*>(&tile[tile_off<D>(key, 2 * c)]) = lo;
    *reinterpret_cast<u32x4_t*>(&tile[tile_off<D>(key, 2 * c + 1)]) = hi;
  };
  auto store_tile = [&](uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int key = 16 * wave + KPI * j + kr0;
      store8(kd, key, pos, kr[j]);
      store8(vd, key, pos, vr[j]);
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

  // lane constants of the operand reads: S^T reads chunk 2 ks + hf of rows
  // col and 32 + col (same permutation); V^T reads (see below) rows
  // tr_c + 4 hf + 8 e (+ multiples of 16) at element 16 tr_g + 4 tr_a + 32 b
  const int kswz = 8 * (hf ^ chunk_swz<D>(col));
  const int tr_a = lane & 3, tr_c = (lane >> 2) & 3, tr_g = (lane >> 4) & 1;
  auto vt_off = [&](int e, int b) __attribute__((always_inline)) {
    const int r = tr_c + 4 * hf + 8 * e;
    return tile_off<D>(r, 4 * b + 2 * tr_g + (tr_a >> 1)) + 4 * (tr_a & 1);
  };

  // S^T[key][query] of one key tile from LDS tile K, for the two 32-key
  // halves of the tile and each query block.  The accumulations are
  // independent: their MFMAs alternate, every K operand read from LDS feeds
  // all query blocks, and the next k-step's K operands are read before this
  // step's MFMAs issue.
  auto qk = [&](const uint16_t* K, f32x16_t (&s)[kQB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
    const uint16_t* krow0 = &K[col * D];
    const uint16_t* krow1 = &K[(32 + col) * D];
    auto kread = [&](const uint16_t* row, int ks) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint4*>(row + (kswz ^ (16 * ks)));
    };
    uint4 ka0 = kread(krow0, 0);
    uint4 ka1 = kread(krow1, 0);
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      uint4 kn0 = ka0, kn1 = ka1;
      if (ks + 1 < DS) {
        kn0 = kread(krow0, ks + 1);
        kn1 = kread(krow1, ks + 1);
      }
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        s[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka0), as_bf16x8(qreg[qb][ks]), s[qb][0], 0, 0, 0);
        s[qb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka1), as_bf16x8(qreg[qb][ks]), s[qb][1], 0, 0, 0);
      }
      ka0 = kn0;
      ka1 = kn1;
    }
  };
  // Mask and tile maximum (scaled, log2 units, both lane halves) of query
  // block qb in tile t.  Register r of half kb holds key
  // n0 + 32 kb + 8 (r / 4) + 4 hf + r % 4; a key is visible iff its offset
  // 32 kb + 8 (r / 4) + r % 4 is at most `lim` (one compare per score, on
  // tiles that reach past the query block's first query only; MASK = false
  // asserts that no key of the tile needs it).
  auto tile_max = [&](auto maskc, f32x16_t (&s)[kQB][2], const int t, const int qb) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    const int n0 = t * kKeys;
    const int qpos = ctx + qw + 32 * qb + col;     // absolute position of the lane's query
    const int lim = (CAUSAL ? qpos : kv_len - 1) - n0 - 4 * hf;
    const bool need_mask = MASK && n0 + kKeys - 1 > (CAUSAL ? ctx + qw + 32 * qb : kv_len - 1);
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
    return fmaxf(mt, __shfl_xor(mt, 32)) * scale;
  };
  // The running maximum is raised only when the tile's exceeds it by more
  // than kSlack; the sum and the output are rescaled then.
  auto rescale = [&](const int qb, const float mt) __attribute__((always_inline)) {
    if (mt > m[qb] + kSlack) {
      const float alpha = fast_exp2(m[qb] - mt);
      l[qb] *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][b][r] *= alpha;
      m[qb] = mt;
    }
  };
  // P^T in bf16: B operand slots s of lane half hf <-> registers 8 ks + s;
  // weights are exp2(score * scale - m), and their bf16 values are summed.
  auto exp_pack = [&](const f32x16_t (&s)[kQB][2], uint32_t (&pb)[kQB][2][2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
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
  };
  // O^T[d][query] += V^T[d][key] P^T[key][query]; slot s of lane half hf in
  // step (kb, ks) is key 32 kb + 16 ks + 8 (s / 4) + 4 hf + s % 4.  The V^T
  // operand (lane: d = 32 b + col) comes from row-major V with transposing
  // reads: in each 16-lane group (d = dg .. dg + 15), lane a + 4 c points at
  // V[key0 + c][dg + 4 a], which hands lane j the 4 keys of d = dg + j.
  auto pv = [&](const uint16_t* V, const uint32_t (&pb)[kQB][2][2][4]) __attribute__((always_inline)) {
    auto read_vt = [&](int step, int b) __attribute__((always_inline)) {
      const int kb = step >> 1, ks = step & 1;
      const uint16_t* src = V + (32 * kb + 16 * ks) * D;
      const uint2 lo = lds_read_tr16(src + vt_off(0, b));
      const uint2 hi = lds_read_tr16(src + vt_off(1, b));
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
  };

  // One key tile from LDS tiles K / V, its phases one after another.
  auto compute = [&](const int t, const uint16_t* K, const uint16_t* V) __attribute__((always_inline)) {
    f32x16_t s[kQB][2];
    qk(K, s);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) rescale(qb, tile_max(std::true_type(), s, t, qb));
    uint32_t pb[kQB][2][2][4];
    exp_pack(s, pb);
    pv(V, pb);
  };

  // Tile t from buffer BUF, the next one into the other buffer.  bf16: the
  // next tile's loads go straight to LDS at the start; E4M3: the staged
  // codes of the next tile are converted into LDS at the end and the loads
  // of the one after are issued.  The barrier (which also waits for this
  // wave's loads into LDS) ends the step.
  auto step = [&](auto bufc, const int t) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    uint16_t* const kd = BUF ? s_k0 : s_k1;
    uint16_t* const vd = BUF ? s_v0 : s_v1;
    if constexpr (!F8) {
      fetch_entries(t + 2, ent_next);
      advance_window(t + 1);
      if (t + 1 < n_tiles) load_tile(t + 1, kd, vd);
    }
    compute(t, BUF ? s_k1 : s_k0, BUF ? s_v1 : s_v0);
    if constexpr (F8) {
      store_tile(kd, vd);
      advance_window(t + 2);
      issue_loads(t + 2);
      fetch_entries(t + 3, ent);
    }
    __syncthreads();
    if constexpr (!F8 && !BIG) {
#pragma unroll
      for (int j = 0; j < NI; ++j) ent[j] = ent_next[j];
    }
  };

  if constexpr (BIG) {
    tab = load_window(0);
    if (64 < n_tiles) tab_next = load_window(64);
  }
  fetch_entries(0, ent);
  if constexpr (F8) {
    issue_loads(0);
    fetch_entries(1, ent);
    store_tile(s_k0, s_v0);
    issue_loads(1);
    fetch_entries(2, ent);
  } else {
    load_tile(0, s_k0, s_v0);
    fetch_entries(1, ent);
  }

  // Software-pipelined tiles (bf16 caches): the leading tiles whose keys
  // every query of the work-group sees need no mask, and for them step t
  // runs the QK^T MFMAs of tile t + 1 beside the exponentials of tile t, and
  // the PV MFMAs of tile t beside the maximum of tile t + 1, so that the
  // matrix cores and the vector ALUs work at the same time.  K runs one tile
  // ahead of V: step t reads K(t + 1) and V(t) and loads K(t + 2) and
  // V(t + 1), each into the buffer of its own parity, which the previous
  // step finished reading.  The remaining (masked) tiles take the plain
  // steps above.
  int t_first = 0;
  if constexpr (!F8) {
    static_assert(kQB == 1, "the pipelined steps hold one query block per wave");
    const int n_pipe = ((CAUSAL ? ctx + q0 : kv_len - 1) + 1) / kKeys;  // tiles without a mask
    if (n_pipe >= 2) {
      // V(t) is loaded one step after K(t), from the same rows: B >= 16
      // keeps the wave's row base, B < 16 the lanes' offsets (and `ent`
      // holds the table entries of the tile whose K is loaded next).
      struct KeyOffs {
        KeyOff off[NI];
      };
      using Addr = typename std::conditional<BIG, Rows, KeyOffs>::type;
      auto tile_addr = [&](int tile) __attribute__((always_inline)) {
        if constexpr (BIG) {
          return tile_rows(tile);
        } else {
          KeyOffs k;
#pragma unroll
          for (int j = 0; j < NI; ++j) k.off[j] = key_off(tile, j);
          return k;
        }
      };
      auto load_addr = [&](const char* cache, const Addr& ad, uint16_t* dst, auto wholec) __attribute__((always_inline)) {
        if constexpr (BIG) {
          load_rows(cache, ad, dst, wholec);
        } else {
#pragma unroll
          for (int j = 0; j < NI; ++j) load_to_lds16(cache + ad.off[j], dst + (16 * wave + KPI * j) * D);
        }
      };
      advance_window(1);
      Addr vaddr = tile_addr(1);           // rows of the tile whose V is loaded next
      load_addr(kcb, vaddr, s_k1, std::false_type());
      fetch_entries(2, ent);
      __syncthreads();
      f32x16_t sc[kQB][2];
      qk(s_k0, sc);
      rescale(0, tile_max(std::false_type(), sc, 0, 0));
      __syncthreads();   // K(0) is read: its buffer takes K(2) next
      // step t: K(t + 1) in buffer (t + 1) & 1, V(t) in buffer t & 1
      auto pstep = [&](auto parc, const int t) __attribute__((always_inline)) {
        constexpr int PAR = decltype(parc)::value;   // t & 1
        uint16_t* const k_next = PAR ? s_k0 : s_k1;  // holds K(t + 1)
        uint16_t* const k_free = PAR ? s_k1 : s_k0;  // K(t) was read last step
        uint16_t* const v_cur = PAR ? s_v1 : s_v0;   // holds V(t)
        uint16_t* const v_free = PAR ? s_v0 : s_v1;  // V(t - 1) was read last step
        load_addr(vcb, vaddr, v_free, std::true_type());   // t + 1 < n_pipe: no key past the end
        if (t + 2 < n_tiles) {
          advance_window(t + 2);
          vaddr = tile_addr(t + 2);
          load_addr(kcb, vaddr, k_free, std::false_type());
        }
        fetch_entries(t + 3, ent);
        f32x16_t sn[kQB][2];
        uint32_t pb[kQB][2][2][4];
        qk(k_next, sn);
        exp_pack(sc, pb);
        pv(v_cur, pb);
        const float mt = tile_max(std::false_type(), sn, t + 1, 0);
        __syncthreads();
        rescale(0, mt);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[0][kb] = sn[0][kb];
      };
      int t = 0;
      for (; t + 2 < n_pipe; t += 2) {
        pstep(std::integral_constant<int, 0>(), t);
        pstep(std::integral_constant<int, 1>(), t + 1);
      }
      if (t + 1 < n_pipe) {
        pstep(std::integral_constant<int, 0>(), t);
        ++t;
      }
      // last pipelined tile t = n_pipe - 1: K(t + 1) is loading (if any);
      // its V goes to the buffer of V(t - 1), then the plain steps go on
      // from t + 1 with tile t + 1 whole in buffer (t + 1) & 1 (and, B < 16,
      // the entries of tile t + 2 in `ent`)
      if (t + 1 < n_tiles) load_addr(vcb, vaddr, (t & 1) ? s_v0 : s_v1, std::false_type());
      uint32_t pb[kQB][2][2][4];
      exp_pack(sc, pb);
      pv((t & 1) ? s_v1 : s_v0, pb);
      __syncthreads();
      t_first = t + 1;
    } else {
      __syncthreads();
    }
  } else {
    __syncthreads();
  }
  int t = t_first;
  if (t & 1) {
    if (t < n_tiles) step(std::integral_constant<int, 1>(), t);
    ++t;
  }
  for (; t < n_tiles; t += 2) {
    step(std::integral_constant<int, 0>(), t);
    if (t + 1 < n_tiles) step(std::integral_constant<int, 1>(), t + 1);
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

}  // namespace prefill_body
}  // namespace pa
