// Paged decode partition pass for gfx950, shared by the decode kernels and
// the mixed-batch kernel (see paged_decode.hip for the design).
#pragma once

#include <type_traits>

#include "../internal.hpp"
#include "common.hpp"

namespace pa {
namespace decode_body {

// Waves of a head-layout work-group: E4M3 caches with at most 4 query heads
// per KV head take 8 (their registers leave room for four waves per SIMD, so
// two 8-wave work-groups share a CU); every other case 4.
template <bool F8, int G>
constexpr int kWaves = F8 && G <= 4 ? 8 : 4;
constexpr int kHalf = 16;     // tokens of a half tile, inside one block when B >= 16
constexpr int kBuffers = 2;   // register buffers per wave (tiles in flight + 1)
constexpr int kHalves8 = 1;   // half tiles per tile with E4M3 rows (bf16: 1)
constexpr int kChunk = 512;   // tokens whose table entries are staged at once (B < 16)
template <int G>
constexpr int kRowBuffers = G <= 4 ? 3 : 2;   // row layout: steps in flight + 1
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;  // log2 units

// Lane layout.  A token's K (or V) row of one KV head is held by LPT = D / 8
// lanes, 8 elements each (lane li = lane % LPT holds d = 8 li .. 8 li + 7:
// one 16-byte piece of bf16, or 8 E4M3 codes), so a lane group reads the
// row's contiguous bytes.  The NG = 64 / LPT groups of a wave hold NG
// consecutive tokens per load instruction; a half tile's 16 tokens take
// TPL = 16 / NG loads, token u of group grp being t0 + grp + NG u.
template <int D>
struct Layout {
  static constexpr int LPT = D / 8;
  static constexpr int NG = 64 / LPT;
  static constexpr int TPL = kHalf / NG;
};

template <bool F8>
using PieceOf = typename std::conditional<F8, uint2, uint4>::type;

// A lane's pieces of the K and V rows of its NT tokens.
template <bool F8, int NT>
struct KV {
  PieceOf<F8> k[NT];
  PieceOf<F8> v[NT];
};

// The 8 elements of a piece as 4 packed bf16 pairs in element order (E4M3
// codes are converted exactly).
template <bool F8>
__device__ __forceinline__ void bf16_words(const PieceOf<F8>& piece, uint32_t (&w)[4]) {
  if constexpr (F8) {
    w[0] = e4m3x2_to_bf16x2<false>(piece.x);
    w[1] = e4m3x2_to_bf16x2<true>(piece.x);
    w[2] = e4m3x2_to_bf16x2<false>(piece.y);
    w[3] = e4m3x2_to_bf16x2<true>(piece.y);
  } else {
    w[0] = piece.x;
    w[1] = piece.y;
    w[2] = piece.z;
    w[3] = piece.w;
  }
}

// One reduce-scatter step over lane pairs that differ in one bit of li:
// a lane whose bit is set keeps the upper half of its values, its partner
// the lower half, and each adds the partner's copy of the half it keeps.
template <int CTRL, int N>
__device__ __forceinline__ void rs_step(const float (&v)[N], float (&w)[N / 2], bool bit) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = bit ? v[k] : v[k + N / 2];
    const float keep = bit ? v[k + N / 2] : v[k];
    w[k] = keep + dpp<CTRL>(send);
  }
}

// Sum of LPT per-lane values over the LPT lanes of a group, scattered: lane
// li of the group ends with the total of value li.  The partner of each step
// flips one bit of li: the row mirror (li <-> 15 - li) bit 3, the half-row
// mirror (li <-> li ^ 7) bit 2, then xor 2 and xor 1.
template <int LPT>
__device__ __forceinline__ float reduce_scatter(const float (&v)[LPT], int li) {
  float w8[8];
  if constexpr (LPT == 16) {
    rs_step<kDppRowMirror>(v, w8, (li & 8) != 0);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) w8[k] = v[k];
  }
  float w4[4], w2[2], w1[1];
  rs_step<kDppHalfMirror>(w8, w4, (li & 4) != 0);
  rs_step<kDppXor2>(w4, w2, (li & 2) != 0);
  rs_step<kDppXor1>(w2, w1, (li & 1) != 0);
  return w1[0];
}

// Each head of a set of four holds one value per token pair in the lanes of
// that pair (group lanes TPL h + 2 q and TPL h + 2 q + 1, q < TPL / 2); every
// lane of the group gets all of them: out[h][q].
template <int TPL>
__device__ __forceinline__ void broadcast_pairs(uint32_t x, int li, uint32_t (&out)[4][TPL / 2]) {
  if constexpr (TPL == 4) {
    // a group is a 16-lane row: broadcast lanes 0, 2, 4, ..., 14 of the row
    out[0][0] = dpp<kDppRowBcast0 + 0>(x);
    out[0][1] = dpp<kDppRowBcast0 + 2>(x);
    out[1][0] = dpp<kDppRowBcast0 + 4>(x);
    out[1][1] = dpp<kDppRowBcast0 + 6>(x);
    out[2][0] = dpp<kDppRowBcast0 + 8>(x);
    out[2][1] = dpp<kDppRowBcast0 + 10>(x);
    out[3][0] = dpp<kDppRowBcast0 + 12>(x);
    out[3][1] = dpp<kDppRowBcast0 + 14>(x);
  } else {
    // a group is half a row (lanes 2h, 2h + 1 hold head h): quad broadcasts
    // give heads 0-1 of this quad, the half-row mirror those of the other
    const bool up4 = (li & 4) != 0;
    const uint32_t a = dpp<kDppBcast0>(x), b = dpp<kDppBcast2>(x);
    const uint32_t a2 = dpp<kDppHalfMirror>(a), b2 = dpp<kDppHalfMirror>(b);
    out[0][0] = up4 ? a2 : a;
    out[1][0] = up4 ? b2 : b;
    out[2][0] = up4 ? a : a2;
    out[3][0] = up4 ? b : b2;
  }
}

// One half tile of a lane: TPL tokens whose K and V pieces are
// r.k / r.v [base + u] (u < TPL); valid: the token of this lane's score lies
// inside the range.  Scores of the lane group's 4 heads x TPL tokens are
// reduce-scattered, one per lane; the running maxima are raised on a rare
// slow path (ROW_MAX: each 16-lane row has its own KV head, so its maxima are
// its own; otherwise every lane group of the wave shares them); the bf16
// weights are paired over tokens and the V pieces accumulated into acc.
template <int D, int G, bool F8, bool ROW_MAX, typename KVt>
__device__ __forceinline__ void attend(const KVt& r, const int base, const bool valid, const uint4 (&qr)[G],
                                       const float scale, float (&m_own)[(G + 3) / 4], float (&l_own)[(G + 3) / 4],
                                       float (&acc)[G][8], const int li) {
  using Lay = Layout<D>;
  constexpr int LPT = Lay::LPT, TPL = Lay::TPL;
  constexpr int NSET = (G + 3) / 4;
  static_assert(!ROW_MAX || TPL == 4, "a row's own maxima need the row to hold one KV head");
  const int my_h = li / TPL;
  const bool b0 = (li & 1) != 0;
  // partial dots: value h TPL + u of set j is head 4 j + h, token u
  float x[NSET];
  {
    uint32_t kw[TPL][4];
#pragma unroll
    for (int u = 0; u < TPL; ++u) bf16_words<F8>(r.k[base + u], kw[u]);
#pragma unroll
    for (int j = 0; j < NSET; ++j) {
      float w[LPT];
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4)
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
          const int h = 4 * j + h4;
          float d = 0.f;
          if (h < G) {
            const uint32_t* qq = reinterpret_cast<const uint32_t*>(&qr[h]);
#pragma unroll
            for (int jw = 0; jw < 4; ++jw) d = dot2_bf16(qq[jw], kw[u][jw], d);
          }
          w[h4 * TPL + u] = d;
        }
      // the reduction is a cross-lane operation: every lane must take
      // part, so it runs unconditionally and invalid slots are masked
      // afterwards
      const float xs = reduce_scatter<LPT>(w, li) * scale;
      const bool ok = (4 * j + my_h < G) && valid;
      x[j] = ok ? xs : kNegInf;
    }
  }
  // rare slow path: raise the running maxima
  bool need = false;
#pragma unroll
  for (int j = 0; j < NSET; ++j) need |= x[j] > m_own[j] + kRescaleSlack;
  if (__any(need)) {
    uint32_t al[NSET][4][1];
#pragma unroll
    for (int j = 0; j < NSET; ++j) {
      // maximum over the lanes holding the same head: its tokens in the
      // group, then (unless ROW_MAX) the groups of the wave
      float mx = x[j];
      mx = fmaxf(mx, dpp<kDppXor1>(mx));
      if constexpr (TPL == 4) {
        mx = fmaxf(mx, dpp<kDppXor2>(mx));
      } else {
        mx = fmaxf(mx, dpp<kDppRor8>(mx));
      }
      if constexpr (!ROW_MAX) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
      }
      const float mn = fmaxf(m_own[j], mx);
      const float alpha = mn == kNegInf ? 1.f : fast_exp2(m_own[j] - mn);
      l_own[j] *= alpha;
      m_own[j] = mn;
      uint32_t al2[4][TPL / 2];
      broadcast_pairs<TPL>(__float_as_uint(alpha), li, al2);
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4) al[j][h4][0] = al2[h4][0];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float alpha = __uint_as_float(al[h >> 2][h & 3][0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] *= alpha;
    }
  }
  // weights: one exponential per lane, paired over tokens (u, u + 1) of a
  // head, broadcast to the group
  uint32_t pp[NSET][4][TPL / 2];
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    const float p = x[j] == kNegInf ? 0.f : fast_exp2(x[j] - m_own[j]);
    const float other = dpp<kDppXor1>(p);
    const uint32_t pk = pack_bf16x2(b0 ? other : p, b0 ? p : other);
    l_own[j] += b0 ? bf16_hi(pk) : bf16_lo(pk);
    broadcast_pairs<TPL>(pk, li, pp[j]);
  }
  // V rows of each token pair interleaved per d: (v0[d], v1[d]) pairs.
#pragma unroll
  for (int q2 = 0; q2 < TPL / 2; ++q2) {
    uint32_t v0[4], v1[4];
    bf16_words<F8>(r.v[base + 2 * q2], v0);
    bf16_words<F8>(r.v[base + 2 * q2 + 1], v1);
#pragma unroll
    for (int jw = 0; jw < 4; ++jw) {
      const uint32_t lo = __builtin_amdgcn_perm(v1[jw], v0[jw], 0x05040100u);
      const uint32_t hi = __builtin_amdgcn_perm(v1[jw], v0[jw], 0x07060302u);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t w = pp[h >> 2][h & 3][q2];
        acc[h][2 * jw] = dot2_bf16(w, lo, acc[h][2 * jw]);
        acc[h][2 * jw + 1] = dot2_bf16(w, hi, acc[h][2 * jw + 1]);
      }
    }
  }
}

// Appending decode (APP): one new token per sequence of the launch, its slot
// and position in the kernel arguments (up to kAppendRows sequences per
// launch).  Every work-group of sequence s takes the sequence's length
// (position + 1) and the block of the new position's table entry (slot / B)
// from these arguments and reads the new token's K/V from the input rows, so
// it never reads a table entry, length or cache row that this launch writes;
// the work-group of the partition holding the new token writes its head's
// K/V rows to the slot, and the one of head 0 also the table entry and the
// length.  The result is that of the cache write with the table update
// followed by decode, in one launch.
constexpr int kAppendRows = 256;
struct AppendRows {
  int64_t slots[kAppendRows];
  int32_t pos[kAppendRows];
};
struct NoAppend {
  int32_t unused;
};
template <bool APP>
using RowsOf = typename std::conditional<APP, AppendRows, NoAppend>::type;

// The partition pass of work-group (partition part, KV head g, sequence s);
// every work-group runs it with 64 W threads (W waves).
template <int D, int G, bool BIG, bool F8, bool APP, int W = kWaves<F8, G>>
__device__ __forceinline__ void decode_partition(const DecodeArgs& a, const RowsOf<APP>& rows, const int part,
                                                 const int g, const int s) {
  using T = typename std::conditional<F8, uint8_t, uint16_t>::type;  // cache element
  using Lay = Layout<D>;
  constexpr int LPT = Lay::LPT, NG = Lay::NG, TPL = Lay::TPL;
  constexpr int NH = F8 ? kHalves8 : 1;   // half tiles per tile
  constexpr int kTile = kHalf * NH;       // tokens per wave iteration
  using KVt = KV<F8, TPL * NH>;
  using P = PieceOf<F8>;
  constexpr int NSET = (G + 3) / 4;        // sets of 4 heads: one score per lane per set
  __shared__ int32_t s_bt[BIG ? 1 : kChunk];
  __shared__ __attribute__((aligned(16))) float s_acc[W][G][D];
  __shared__ float s_l[W][G];
  __shared__ float s_m[W][G];

  static_assert(!(APP && F8), "appending decode takes bf16 caches");
  static_assert(LPT == 4 * TPL, "a group reduces 4 heads x TPL tokens, one value per lane");
  // (an appending launch of rows r0 .. r0 + n - 1 gets every per-sequence
  // array offset by r0 on the host, so that no address waits for a load)
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (SGPR) so that the tile loop below branches on scalars
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane / LPT, li = lane % LPT, row = lane >> 4;
  const int my_h = li / TPL, my_u = li % TPL;   // the (head in set, token) whose score this lane finishes

  const int P_ = a.partition_size;
  const int start = part * P_;
  const int lgB = a.log2_block_size;
  const int Bmask = (1 << lgB) - 1;
  const int64_t row_elems = (int64_t)a.num_kv_heads * D;
  const int64_t bstride = a.cache_block_stride;
  const T* kcache = static_cast<const T*>(a.key_cache);
  const T* vcache = static_cast<const T*>(a.value_cache);
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.bt_stride;
  const int width = (a.max_seq_len + Bmask) >> lgB;   // table entries that may be read
  const float scale = a.scale * kLog2e;

  // APP: this sequence's new token (position, slot) and the block its
  // position's table entry names after the append
  int64_t app_slot = -1;
  int app_pos = -1;
  if constexpr (APP) {
    app_slot = rows.slots[s];
    app_pos = rows.pos[s];
  }
  const bool app = APP && app_slot >= 0;
  const int app_j = app ? app_pos >> lgB : -1;
  const int app_blk = app ? (int)(app_slot >> lgB) : 0;
  // table entry j as the kernel sees it (APP: the new position's entry from
  // the arguments).  Prefetched entries are loaded as they stand and fixed
  // where they are used, so that their loads never wait for the position.
  auto fix_entry = [&](int j, int b) __attribute__((always_inline)) {
    return APP && j == app_j ? app_blk : b;
  };
  auto entry = [&](int j) __attribute__((always_inline)) { return fix_entry(j, bt_row[j]); };

  // Independent loads first: the length, the queries and (B < 16) the first
  // chunk's table entries, so that their latencies overlap.
  int len = a.seq_lens[s];
  if (app) len = app_pos + 1;
  uint4 qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                            ((int64_t)s * a.num_q_heads + g * G + h) * D + 8 * li);
  auto stage_table = [&](int c0) {
    const int j0 = c0 >> lgB;
    int nj = ((c0 + kChunk - 1) >> lgB) - j0 + 1;
    nj = nj < width - j0 ? nj : width - j0;
    for (int i = tid; i < nj; i += 64 * W) {
      int b = entry(j0 + i);
      b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
      s_bt[i] = b;
    }
  };
  if (!BIG) stage_table(start);
  // BIG: the table entries of the halves of this wave's first two tiles and
  // of the partition's first token, fetched before the length is known
  // (indexes are kept inside the row), so that the first K/V loads wait for
  // one round trip instead of two.
  int pre[2][NH] = {}, pre_start = 0;
  if constexpr (BIG) {
    const int wmax = width - 1;
    const int tw = start + wave * kTile;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const int i = (tw + k * W * kTile + hf * kHalf) >> lgB;
        pre[k][hf] = bt_row[i < wmax ? i : wmax];
      }
    const int is = start >> lgB;
    pre_start = bt_row[is < wmax ? is : wmax];
  }

  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  // A partition past the sequence's last one gets an empty range and returns
  // before the merge; there is no early exit here, which would let the
  // compiler move the table loads above behind it.
  const bool live = part * P_ < len || part == 0;
  const int end = !live ? start : (start + P_ < len ? start + P_ : len);

  // per-lane constant part of a K/V element offset
  const int lane_off = g * D + 8 * li;

  // APP: the new token's K/V rows of this head in the input, and their copy
  // into the cache by the partition that holds the new position
  // (lanes 0 .. 2 D / 8 - 1 of wave 0 copy one 16-byte piece each: the piece
  // is loaded here and stored after the merge, so that the store neither
  // waits for the load nor holds up the wave's first K/V loads)
  const T* new_k = nullptr;
  const T* new_v = nullptr;
  bool app_copy = false;
  uint4 app_piece = make_uint4(0, 0, 0, 0);
  if constexpr (APP) {
    new_k = static_cast<const T*>(a.new_key) + (int64_t)s * a.new_key_stride + g * D;
    new_v = static_cast<const T*>(a.new_value) + (int64_t)s * a.new_value_stride + g * D;
    app_copy = app && app_pos / P_ == part && wave == 0 && lane < 2 * (D / 8);
    if (app_copy) app_piece = *reinterpret_cast<const uint4*>((lane < D / 8 ? new_k : new_v) + 8 * (lane % (D / 8)));
  }

  float m_own[NSET], l_own[NSET], acc[G][8];
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    m_own[j] = kNegInf;
    l_own[j] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;

  // Tokens c0 .. c1 - 1 (B < 16: their table entries are in LDS from j0 on).
  auto range = [&](const int c0, const int c1, const int j0) __attribute__((always_inline)) {

    // Tokens past c1 read token c0 (always valid), so every load stays inside
    // the cache and can be issued unconditionally: with no branch around the
    // prefetches the compiler's wait counts stay exact and the next tiles'
    // loads remain in flight while this one is computed.  All K loads are
    // issued before the V loads so q.k can start first.
    // (with `fetched`, the block ids are `pf`, fetched early for tile t0, or
    // pre_start for a half past c1)
    auto load = [&](int t0, KVt& r, bool fetched = false, const int* pf = nullptr) __attribute__((always_inline)) {
      const T* kp[NH * TPL];
      const T* vp[NH * TPL];
      if (BIG) {
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
          const int th = t0 + hf * kHalf;
          const int tc = th < c1 ? th : c0;          // wave-uniform
          int blk = __builtin_amdgcn_readfirstlane(fetched ? fix_entry(tc >> lgB, th < c1 ? pf[hf] : pre_start)
                                                           : entry(tc >> lgB));
          blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
          const int64_t base = (int64_t)blk * bstride + (int64_t)(tc & Bmask) * row_elems;
          // tokens past c1 read the half's first token (valid): their slots
          // may hold anything, and a zero weight times a NaN is NaN
#pragma unroll
          for (int u = 0; u < TPL; ++u) {
            const int r_ = tc + grp + NG * u < c1 ? grp + NG * u : 0;
            const int64_t off = r_ * row_elems + lane_off;
            const bool isnew = APP && app && tc + r_ == app_pos;
            kp[hf * TPL + u] = isnew ? new_k + 8 * li : kcache + base + off;
            vp[hf * TPL + u] = isnew ? new_v + 8 * li : vcache + base + off;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NH * TPL; ++i) {
          int t = t0 + (i / TPL) * kHalf + grp + NG * (i % TPL);
          t = t < c1 ? t : c0;
          const int64_t blk = s_bt[(t >> lgB) - j0];
          const int64_t off = blk * bstride + (int64_t)(t & Bmask) * row_elems + lane_off;
          const bool isnew = APP && app && t == app_pos;
          kp[i] = isnew ? new_k + 8 * li : kcache + off;
          vp[i] = isnew ? new_v + 8 * li : vcache + off;
        }
      }
#pragma unroll
      for (int i = 0; i < NH * TPL; ++i) r.k[i] = *reinterpret_cast<const P*>(kp[i]);
#pragma unroll
      for (int i = 0; i < NH * TPL; ++i) r.v[i] = *reinterpret_cast<const P*>(vp[i]);
    };

    // One half tile: tokens t0 + grp + NG u of each group, held in
    // r.k / r.v [TPL hf + u].
    auto compute = [&](int t0, const KVt& r, const int hf) __attribute__((always_inline)) {
      attend<D, G, F8, false>(r, TPL * hf, t0 + grp + NG * my_u < c1, qr, scale, m_own, l_own, acc, li);
    };

    // kBuffers register buffers: while tile t is computed, the next
    // kBuffers - 1 tiles of the wave are in flight.  The loop runs whole
    // rounds of kBuffers tiles and has a single, bottom-tested exit (an exit
    // in the middle gives the compiler a path back into the loop with loads
    // pending, and it then drains every load at the top); the last tiles are
    // computed after it from buffers already loaded.  All branches here are
    // wave-uniform.  The first loads are issued whatever n_tiles is (they
    // stay inside the cache), so nothing delays them.
    constexpr int kStep = W * kTile;
    constexpr int NB = kBuffers;
    int t = c0 + wave * kTile;
    const int n_tiles = t < c1 ? (c1 - t + kStep - 1) / kStep : 0;
    KVt r[NB];
#pragma unroll
    for (int k = 0; k + 1 < NB; ++k) load(t + k * kStep, r[k], BIG && k < 2, pre[k < 2 ? k : 0]);
    int i = 0;
    for (; i + NB <= n_tiles; i += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        load(t + (NB - 1) * kStep, r[(k + NB - 1) % NB]);
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) compute(t + hf * kHalf, r[k], hf);
        t += kStep;
      }
    }
#pragma unroll
    for (int k = 0; k + 1 < NB; ++k)
      if (n_tiles - i > k) {
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) compute(t + k * kStep + hf * kHalf, r[k], hf);
      }
  };
  if constexpr (BIG) {
    // one range: no outer loop, whose header would drain the query loads
    // before the first K/V loads are issued
    range(start, end, start >> lgB);
  } else {
    for (int c0 = start; c0 < end; c0 += kChunk) {
      if (c0 != start) {
        __syncthreads();
        stage_table(c0);
      }
      __syncthreads();
      range(c0, c0 + kChunk < end ? c0 + kChunk : end, c0 >> lgB);
    }
  }

  if (!live) return;
  const int nparts = len > 0 ? (len + P_ - 1) / P_ : 1;

  // Merge.  All lane groups of a wave share the running maxima, so their
  // partial sums add directly: (D = 64) the two groups of each 16-lane row
  // with DPP, then the four rows in registers with gfx950's lane swaps, then
  // the W waves through LDS.  permlane32_swap(x, y) exchanges lanes 32..63
  // of x with lanes 0..31 of y, permlane16_swap(x, y) the odd 16-lane rows of
  // x with the even rows of y; adding the two results of a swap sums rows
  // (0, 2) and (1, 3), then rows 0 and 1.  With the lane's NV sums flattened
  // as v = 8 h + i and paired as below, row r ends with the totals of
  // v = r Q .. r Q + Q - 1 (D = 64: in lanes 0..7 of the row, copies in 8..15).
  constexpr int NV = G * 8;
  constexpr int Q = NV / 4;
  float xs[NV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[h * 8 + i] = LPT == 16 ? acc[h][i] : acc[h][i] + dpp<kDppRor8>(acc[h][i]);
  auto swap_add32 = [](float x, float y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
  auto swap_add16 = [](float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
  float tot[Q];
#pragma unroll
  for (int m = 0; m < Q; ++m) {
    // pair 2m = (v m, v 2Q + m) and pair 2m + 1 = (v Q + m, v 3Q + m): after
    // the 32-lane step each holds its first value in rows 0-1 and its second
    // in rows 2-3; the 16-lane step then puts v m, Q + m, 2Q + m, 3Q + m in
    // rows 0, 1, 2, 3
    const float a_ = swap_add32(xs[m], xs[2 * Q + m]);
    const float b_ = swap_add32(xs[Q + m], xs[3 * Q + m]);
    tot[m] = swap_add16(a_, b_);
  }
  // l: the lanes of a head in a group (its tokens), then the rows
  float lp[NSET];
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    lp[j] = l_own[j] + dpp<kDppXor1>(l_own[j]);
    if constexpr (TPL == 4) {
      lp[j] += dpp<kDppXor2>(lp[j]);
    } else {
      lp[j] += dpp<kDppRor8>(lp[j]);
    }
    lp[j] = swap_add32(lp[j], lp[j]);
    lp[j] = swap_add16(lp[j], lp[j]);
  }
  if (LPT == 16 || (lane & 8) == 0) {
    if constexpr (Q % 8 == 0) {
      // row r: heads r Q / 8 + c, 8 consecutive elements each
#pragma unroll
      for (int c = 0; c < Q / 8; ++c) {
        const int h = row * (Q / 8) + c;
        float* dst = &s_acc[wave][h][8 * li];
        *reinterpret_cast<float4*>(dst) = make_float4(tot[8 * c], tot[8 * c + 1], tot[8 * c + 2], tot[8 * c + 3]);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(tot[8 * c + 4], tot[8 * c + 5], tot[8 * c + 6], tot[8 * c + 7]);
      }
    } else {
#pragma unroll
      for (int m = 0; m < Q; ++m) {
        const int v = row * Q + m;
        s_acc[wave][v >> 3][8 * li + (v & 7)] = tot[m];
      }
    }
    if (row == 0 && my_u == 0) {
#pragma unroll
      for (int j = 0; j < NSET; ++j) {
        const int h = 4 * j + my_h;
        if (h < G) {
          s_l[wave][h] = lp[j];
          s_m[wave][h] = m_own[j];
        }
      }
    }
  }
  __syncthreads();

  // Combine the waves: thread -> (head h, dim d) outputs.
  for (int o = tid; o < G * D; o += 64 * W) {
    const int h = o / D, d = o % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = s_m[w][h];
        const float e = mw == kNegInf ? 0.f : fast_exp2(mw - M);
        L += s_l[w][h] * e;
        A += s_acc[w][h][d] * e;
      }
    }
    const int hq = g * G + h;
    const int64_t orow = (int64_t)s * a.num_q_heads + hq;
    const float val = L > 0.f ? A / L * a.v_scale : 0.f;
    const float lse2 = L > 0.f ? M + fast_log2(L) : kNegInf;
    if (nparts == 1) {
      static_cast<uint16_t*>(a.out)[orow * D + d] = to_bf16(val);
      if (a.lse && d == 0) a.lse[orow] = lse2 * kLn2;
    } else {
      a.ws_out[(orow * a.max_parts + part) * D + d] = val;
      if (d == 0) a.ws_lse[orow * a.max_parts + part] = lse2;
    }
  }

  // APP: the new token's K/V rows of this head into its slot, and (head 0)
  // the new position's table entry and the length
  if constexpr (APP) {
    if (app_copy) {
      const int c = lane % (D / 8);
      const int64_t dst = (int64_t)app_blk * bstride + (app_slot & Bmask) * row_elems + g * D + 8 * c;
      T* cache = const_cast<T*>(lane < D / 8 ? kcache : vcache);
      *reinterpret_cast<uint4*>(cache + dst) = app_piece;
      if (g == 0 && lane == 0) {
        if (app_j < a.bt_stride) a.wr_tables[(int64_t)s * a.bt_stride + app_j] = app_blk;
        a.wr_lens[s] = app_pos + 1;
      }
    }
  }
}

// Lane 4 h4 of each 16-lane row to the whole row (h4 a compile-time value
// after unrolling).
__device__ __forceinline__ float row_bcast4(float x, int h4) {
  switch (h4) {
    case 0: return dpp<kDppRowBcast0 + 0>(x);
    case 1: return dpp<kDppRowBcast0 + 4>(x);
    case 2: return dpp<kDppRowBcast0 + 8>(x);
    default: return dpp<kDppRowBcast0 + 12>(x);
  }
}

// Row layout (D = 128, bf16 caches, KV heads a multiple of 4): the
// partition pass of one wave, item (head set hs, partition part, sequence s),
// where head set hs is KV heads 4 hs .. 4 hs + 3.  Row r of the wave (lanes
// 16 r .. 16 r + 15) holds KV head 4 hs + r, lane li its elements
// 8 li .. 8 li + 7, so one load instruction reads one token's rows of the
// four heads: 1 KiB of contiguous cache.  The wave walks the partition's
// tokens 4 at a time (lane load u = token t0 + u) with NB - 1 steps of loads
// in flight, and writes its heads' partials itself: no LDS and no barrier,
// so the waves of a work-group are independent.  The work-group's four
// waves take consecutive items (head sets fastest), so the head sets of one
// partition read the same tokens' whole rows at about the same time.
template <int G, bool BIG, bool APP, int NB>
__device__ __forceinline__ void decode_rows(const DecodeArgs& a, const RowsOf<APP>& rows, const int part,
                                            const int hs, const int s) {
  constexpr int D = 128;
  using T = uint16_t;
  using Lay = Layout<D>;
  constexpr int TPL = Lay::TPL;
  using KVt = KV<false, TPL>;
  constexpr int NSET = (G + 3) / 4;
  static_assert(TPL == 4 && NB >= 2, "row layout: 4 tokens per step");
  const int lane = threadIdx.x & 63;
  const int row = lane >> 4, li = lane & 15;
  const int my_h = li / TPL, my_u = li % TPL;   // the (head in set, token) whose score this lane finishes
  const int g = 4 * hs + row;                   // this row's KV head

  const int P_ = a.partition_size;
  const int start = part * P_;
  const int lgB = a.log2_block_size;
  const int Bmask = (1 << lgB) - 1;
  const int64_t row_elems = (int64_t)a.num_kv_heads * D;
  const int64_t bstride = a.cache_block_stride;
  const T* kcache = static_cast<const T*>(a.key_cache);
  const T* vcache = static_cast<const T*>(a.value_cache);
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.bt_stride;
  const int width = (a.max_seq_len + Bmask) >> lgB;
  const float scale = a.scale * kLog2e;

  int64_t app_slot = -1;
  int app_pos = -1;
  if constexpr (APP) {
    app_slot = rows.slots[s];
    app_pos = rows.pos[s];
  }
  const bool app = APP && app_slot >= 0;
  const int app_j = app ? app_pos >> lgB : -1;
  const int app_blk = app ? (int)(app_slot >> lgB) : 0;

  // independent loads first: the length, the queries and the table entry of
  // the partition's first token (index kept inside the row)
  int len = a.seq_lens[s];
  if (app) len = app_pos + 1;
  uint4 qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                            ((int64_t)s * a.num_q_heads + g * G + h) * D + 8 * li);
  int nxt = 0;
  if constexpr (BIG) {
    const int j_start = (start >> lgB) < width - 1 ? (start >> lgB) : width - 1;
    nxt = bt_row[j_start];
  }

  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const bool live = part * P_ < len || part == 0;
  const int end = !live ? start : (start + P_ < len ? start + P_ : len);
  const int lane_off = g * D + 8 * li;

  // APP: this row's pieces of the new token's K/V rows, copied into the slot
  // by the waves of the partition that holds the new position
  const T* new_k = nullptr;
  const T* new_v = nullptr;
  bool app_copy = false;
  uint4 app_k = make_uint4(0, 0, 0, 0), app_v = app_k;
  if constexpr (APP) {
    new_k = static_cast<const T*>(a.new_key) + (int64_t)s * a.new_key_stride + lane_off;
    new_v = static_cast<const T*>(a.new_value) + (int64_t)s * a.new_value_stride + lane_off;
    app_copy = app && app_pos / P_ == part;
    if (app_copy) {
      app_k = *reinterpret_cast<const uint4*>(new_k);
      app_v = *reinterpret_cast<const uint4*>(new_v);
    }
  }

  float m_own[NSET], l_own[NSET], acc[G][8];
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    m_own[j] = kNegInf;
    l_own[j] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;

  // Step t0 (a multiple of 4 from the partition start): tokens past `end`
  // read token tc (valid), steps past `end` read the partition's first
  // token, so every load stays inside the cache and is issued
  // unconditionally.  B >= 16: the step's 4 tokens lie in one block; the
  // steps are loaded in order, and each load fetches the next step's table
  // entry (nxt) for the next call, so the scalar load has a whole step to
  // land.  B < 16: each token's entry is a scalar load of its own (all lanes
  // of a load read the same token).
  auto load = [&](const int t0, KVt& r) __attribute__((always_inline)) {
    const int tc = t0 < end ? t0 : start;
    const T* kp[TPL];
    const T* vp[TPL];
    if constexpr (BIG) {
      int blk = __builtin_amdgcn_readfirstlane(APP && (tc >> lgB) == app_j ? app_blk : nxt);
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      const int t1 = t0 + 4 < end ? t0 + 4 : start;
      nxt = bt_row[t1 >> lgB];
      const int64_t base = (int64_t)blk * bstride + (int64_t)(tc & Bmask) * row_elems + lane_off;
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const int r_ = tc + u < end ? u : 0;
        const bool isnew = APP && app && tc + r_ == app_pos;
        kp[u] = isnew ? new_k : kcache + base + r_ * row_elems;
        vp[u] = isnew ? new_v : vcache + base + r_ * row_elems;
      }
    } else {
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const int tok = tc + u < end ? tc + u : tc;
        const int j = tok >> lgB;
        int blk = __builtin_amdgcn_readfirstlane(APP && j == app_j ? app_blk : bt_row[j]);
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        const int64_t off = (int64_t)blk * bstride + (int64_t)(tok & Bmask) * row_elems + lane_off;
        const bool isnew = APP && app && tok == app_pos;
        kp[u] = isnew ? new_k : kcache + off;
        vp[u] = isnew ? new_v : vcache + off;
      }
    }
#pragma unroll
    for (int u = 0; u < TPL; ++u) r.k[u] = *reinterpret_cast<const uint4*>(kp[u]);
#pragma unroll
    for (int u = 0; u < TPL; ++u) r.v[u] = *reinterpret_cast<const uint4*>(vp[u]);
  };

  // NB register buffers: while step i is computed, steps i + 1 .. i + NB - 1
  // are in flight.  Whole rounds of NB steps with a single bottom-tested
  // exit, then the loaded tail (as in the head layout).
  const int n_steps = (end - start + 3) >> 2;
  KVt r[NB];
  int t = start;
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k) load(t + 4 * k, r[k]);
  int i = 0;
  for (; i + NB <= n_steps; i += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      load(t + 4 * (NB - 1), r[(k + NB - 1) % NB]);
      attend<D, G, false, true>(r[k], 0, t + my_u < end, qr, scale, m_own, l_own, acc, li);
      t += 4;
    }
  }
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k)
    if (n_steps - i > k) attend<D, G, false, true>(r[k], 0, t + 4 * k + my_u < end, qr, scale, m_own, l_own, acc, li);

  if (!live) return;
  const int nparts = len > 0 ? (len + P_ - 1) / P_ : 1;

  // the row's sums of the weights per head (over the head's 4 token lanes);
  // the maxima are already equal on those lanes
  float lsum[NSET];
#pragma unroll
  for (int j = 0; j < NSET; ++j) {
    lsum[j] = l_own[j] + dpp<kDppXor1>(l_own[j]);
    lsum[j] += dpp<kDppXor2>(lsum[j]);
  }
  const int64_t q0 = (int64_t)s * a.num_q_heads + g * G;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float L = row_bcast4(lsum[h >> 2], h & 3);
    float val[8];
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) val[i2] = L > 0.f ? acc[h][i2] / L * a.v_scale : 0.f;
    if (nparts == 1) {
      uint4 o;
      o.x = pack_bf16x2(val[0], val[1]);
      o.y = pack_bf16x2(val[2], val[3]);
      o.z = pack_bf16x2(val[4], val[5]);
      o.w = pack_bf16x2(val[6], val[7]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (q0 + h) * D + 8 * li) = o;
    } else {
      float* dst = a.ws_out + ((q0 + h) * a.max_parts + part) * D + 8 * li;
      *reinterpret_cast<float4*>(dst) = make_float4(val[0], val[1], val[2], val[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(val[4], val[5], val[6], val[7]);
    }
  }
  if (my_u == 0) {
#pragma unroll
    for (int j = 0; j < NSET; ++j) {
      const int h = 4 * j + my_h;
      if (h < G) {
        const float lse2 = lsum[j] > 0.f ? m_own[j] + fast_log2(lsum[j]) : kNegInf;
        if (nparts == 1) {
          if (a.lse) a.lse[q0 + h] = lse2 * kLn2;
        } else {
          a.ws_lse[(q0 + h) * a.max_parts + part] = lse2;
        }
      }
    }
  }

  // APP: the new token's K/V rows of this wave's heads into the slot, and
  // (head set 0) the new position's table entry and the length
  if constexpr (APP) {
    if (app_copy) {
      const int64_t dst = (int64_t)app_blk * bstride + (app_slot & Bmask) * row_elems + lane_off;
      *reinterpret_cast<uint4*>(const_cast<T*>(kcache) + dst) = app_k;
      *reinterpret_cast<uint4*>(const_cast<T*>(vcache) + dst) = app_v;
      if (hs == 0 && lane == 0) {
        if (app_j < a.bt_stride) a.wr_tables[(int64_t)s * a.bt_stride + app_j] = app_blk;
        a.wr_lens[s] = app_pos + 1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// E4M3 row layout (head_dim 128, at most 4 query heads per KV head).  Wave
// item = (head set hs of 4 KV heads, partition, sequence), as in the bf16
// row layout, but a lane holds 16 codes: 16-lane row r holds KV head
// 4 hs + r, its half row hw the tokens of parity hw, and lane c of the half
// row the codes 16 c .. 16 c + 15 of its token's row.  One load instruction
// thus reads the four heads' rows of two consecutive tokens (two runs of
// 512 contiguous bytes), and a step of 8 tokens is 4 loads each of K and V.
constexpr int kRows8Tokens = 8;
constexpr int kRows8Buffers = 2;   // steps in flight + 1

// 8 bf16 pairs (elements 2 j, 2 j + 1) of 16 E4M3 codes (exact conversion).
__device__ __forceinline__ void e4m3x16_words(const uint4& x, uint32_t (&w)[8]) {
  w[0] = e4m3x2_to_bf16x2<false>(x.x);
  w[1] = e4m3x2_to_bf16x2<true>(x.x);
  w[2] = e4m3x2_to_bf16x2<false>(x.y);
  w[3] = e4m3x2_to_bf16x2<true>(x.y);
  w[4] = e4m3x2_to_bf16x2<false>(x.z);
  w[5] = e4m3x2_to_bf16x2<true>(x.z);
  w[6] = e4m3x2_to_bf16x2<false>(x.w);
  w[7] = e4m3x2_to_bf16x2<true>(x.w);
}

// E4M3 row layout: the value of lane 2 h of each 16-lane row (the first
// lane that finishes head h's scores) broadcast to the whole row.
__device__ __forceinline__ float row_bcast_pair(float x, int h) {
  switch (h) {
    case 0: return dpp<kDppRowBcast0 + 0>(x);
    case 1: return dpp<kDppRowBcast0 + 2>(x);
    case 2: return dpp<kDppRowBcast0 + 4>(x);
    default: return dpp<kDppRowBcast0 + 6>(x);
  }
}

// Two tokens of a lane group (the half row): k0/v0 and k1/v1 hold the lane's
// codes of tokens t0 + hw and t0 + 2 + hw.  The group's G heads x 2 tokens
// partial dots are reduce-scattered over its 8 lanes (lane c finishes head
// c / 2, token c % 2); a row's maxima are its own (one KV head per row) and
// are taken over both half rows; the bf16 weights are paired over the two
// tokens and broadcast to the half row, and the V codes accumulated.
template <int G>
__device__ __forceinline__ void attend_e4m3_rows(const uint4& k0, const uint4& k1, const uint4& v0, const uint4& v1,
                                                 const bool valid, const uint32_t (&qw)[G][8], const float scale,
                                                 float& m_own, float& l_own, float (&acc)[G][16], const int c) {
  static_assert(G >= 1 && G <= 4, "E4M3 row layout: at most 4 query heads per KV head");
  float x;
  {
    uint32_t kw[2][8];
    e4m3x16_words(k0, kw[0]);
    e4m3x16_words(k1, kw[1]);
    float w[8];
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float d = 0.f;
        if (h4 < G) {
#pragma unroll
          for (int jw = 0; jw < 8; ++jw) d = dot2_bf16(qw[h4][jw], kw[u][jw], d);
        }
        w[2 * h4 + u] = d;
      }
    const float xs = reduce_scatter<8>(w, c) * scale;
    x = (c / 2 < G && valid) ? xs : kNegInf;
  }
  // rare slow path: raise the row's running maxima
  if (__any(x > m_own + kRescaleSlack)) {
    float mx = fmaxf(x, dpp<kDppXor1>(x));
    mx = fmaxf(mx, dpp<kDppRor8>(mx));
    const float mn = fmaxf(m_own, mx);
    const float alpha = mn == kNegInf ? 1.f : fast_exp2(m_own - mn);
    l_own *= alpha;
    m_own = mn;
    uint32_t al[4][1];
    broadcast_pairs<2>(__float_as_uint(alpha), c, al);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = __uint_as_float(al[h][0]);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] *= ah;
    }
  }
  // weights: one exponential per lane, paired over the two tokens of a head
  const bool b0 = (c & 1) != 0;
  const float p = x == kNegInf ? 0.f : fast_exp2(x - m_own);
  const float other = dpp<kDppXor1>(p);
  const uint32_t pk = pack_bf16x2(b0 ? other : p, b0 ? p : other);
  l_own += b0 ? bf16_hi(pk) : bf16_lo(pk);
  uint32_t pp[4][1];
  broadcast_pairs<2>(pk, c, pp);
  // V rows of the two tokens interleaved per d: (v0[d], v1[d]) pairs
  uint32_t vw0[8], vw1[8];
  e4m3x16_words(v0, vw0);
  e4m3x16_words(v1, vw1);
#pragma unroll
  for (int jw = 0; jw < 8; ++jw) {
    const uint32_t lo = __builtin_amdgcn_perm(vw1[jw], vw0[jw], 0x05040100u);
    const uint32_t hi = __builtin_amdgcn_perm(vw1[jw], vw0[jw], 0x07060302u);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      acc[h][2 * jw] = dot2_bf16(pp[h][0], lo, acc[h][2 * jw]);
      acc[h][2 * jw + 1] = dot2_bf16(pp[h][0], hi, acc[h][2 * jw + 1]);
    }
  }
}

// The partition pass of wave item (partition part, head set hs, sequence s)
// over E4M3 caches; NB register buffers of one step each.
template <int G, bool BIG, int NB>
__device__ __forceinline__ void decode_rows8(const DecodeArgs& a, const int part, const int hs, const int s) {
  constexpr int D = 128;
  constexpr int kT = kRows8Tokens;
  static_assert(NB >= 2, "at least one step in flight");
  const int lane = threadIdx.x & 63;
  const int row = lane >> 4, hw = (lane >> 3) & 1, c = lane & 7;
  const int g = 4 * hs + row;   // this row's KV head

  const int P_ = a.partition_size;
  const int start = part * P_;
  const int lgB = a.log2_block_size;
  const int Bmask = (1 << lgB) - 1;
  const int64_t row_bytes = (int64_t)a.num_kv_heads * D;   // one byte per code
  const int64_t bstride = a.cache_block_stride;
  const uint8_t* kcache = static_cast<const uint8_t*>(a.key_cache);
  const uint8_t* vcache = static_cast<const uint8_t*>(a.value_cache);
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.bt_stride;
  const int width = (a.max_seq_len + Bmask) >> lgB;
  const float scale = a.scale * kLog2e;

  // independent loads first: the length, the queries (the lane's 16
  // elements of each of its KV head's query heads) and the table entry of
  // the partition's first token
  int len = a.seq_lens[s];
  uint32_t qw[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                     ((int64_t)s * a.num_q_heads + g * G + h) * D + 16 * c);
    const uint4 x0 = qp[0], x1 = qp[1];
    qw[h][0] = x0.x;
    qw[h][1] = x0.y;
    qw[h][2] = x0.z;
    qw[h][3] = x0.w;
    qw[h][4] = x1.x;
    qw[h][5] = x1.y;
    qw[h][6] = x1.z;
    qw[h][7] = x1.w;
  }
  int nxt = 0;
  if constexpr (BIG) {
    const int j_start = (start >> lgB) < width - 1 ? (start >> lgB) : width - 1;
    nxt = bt_row[j_start];
  }

  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const bool live = part * P_ < len || part == 0;
  const int end = !live ? start : (start + P_ < len ? start + P_ : len);
  const int lane_off = g * D + 16 * c;

  float m_own = kNegInf, l_own = 0.f, acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;

  struct Step {
    uint4 k[kT / 2];
    uint4 v[kT / 2];
  };
  // Step t0 (a multiple of 8 from the partition start, so with B >= 16 its
  // tokens lie in one block): load u fetches token t0 + 2 u + hw.  Tokens
  // past `end` read the step's first token (valid), steps past `end` the
  // partition's first token, so every load stays inside the cache and is
  // issued unconditionally.  B >= 16: the step's block id was fetched by the
  // previous load (nxt); B < 16: a scalar load per token.
  auto load = [&](const int t0, Step& r) __attribute__((always_inline)) {
    const int tc = t0 < end ? t0 : start;
    const uint8_t* kp[kT / 2];
    const uint8_t* vp[kT / 2];
    if constexpr (BIG) {
      int blk = __builtin_amdgcn_readfirstlane(nxt);
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
      const int t1 = t0 + kT < end ? t0 + kT : start;
      nxt = bt_row[t1 >> lgB];
      const int64_t base = (int64_t)blk * bstride + (int64_t)(tc & Bmask) * row_bytes + lane_off;
#pragma unroll
      for (int u = 0; u < kT / 2; ++u) {
        const int o = 2 * u + hw;
        const int r_ = tc + o < end ? o : 0;
        kp[u] = kcache + base + r_ * row_bytes;
        vp[u] = vcache + base + r_ * row_bytes;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kT / 2; ++u) {
        const int ta = tc + 2 * u < end ? tc + 2 * u : tc;
        const int tb = tc + 2 * u + 1 < end ? tc + 2 * u + 1 : tc;
        int ba = __builtin_amdgcn_readfirstlane(bt_row[ta >> lgB]);
        int bb = __builtin_amdgcn_readfirstlane(bt_row[tb >> lgB]);
        ba = ba < 0 ? 0 : (ba >= a.num_blocks ? a.num_blocks - 1 : ba);
        bb = bb < 0 ? 0 : (bb >= a.num_blocks ? a.num_blocks - 1 : bb);
        const int tok = hw ? tb : ta;
        const int64_t off = (int64_t)(hw ? bb : ba) * bstride + (int64_t)(tok & Bmask) * row_bytes + lane_off;
        kp[u] = kcache + off;
        vp[u] = vcache + off;
      }
    }
#pragma unroll
    for (int u = 0; u < kT / 2; ++u) r.k[u] = *reinterpret_cast<const uint4*>(kp[u]);
#pragma unroll
    for (int u = 0; u < kT / 2; ++u) r.v[u] = *reinterpret_cast<const uint4*>(vp[u]);
  };
  // the lane's score in pair q of step t0 is of token t0 + 4 q + 2 (c % 2) + hw
  auto compute = [&](const int t0, const Step& r) __attribute__((always_inline)) {
#pragma unroll
    for (int q2 = 0; q2 < kT / 4; ++q2)
      attend_e4m3_rows<G>(r.k[2 * q2], r.k[2 * q2 + 1], r.v[2 * q2], r.v[2 * q2 + 1],
                          t0 + 4 * q2 + 2 * (c & 1) + hw < end, qw, scale, m_own, l_own, acc, c);
  };

  // NB register buffers: while step i is computed, steps i + 1 .. i + NB - 1
  // are in flight; whole rounds of NB steps with a single bottom-tested exit,
  // then the loaded tail.
  const int n_steps = (end - start + kT - 1) / kT;
  Step rb[NB];
  int t = start;
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k) load(t + kT * k, rb[k]);
  int i = 0;
  for (; i + NB <= n_steps; i += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      load(t + kT * (NB - 1), rb[(k + NB - 1) % NB]);
      compute(t, rb[k]);
      t += kT;
    }
  }
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k)
    if (n_steps - i > k) compute(t + kT * k, rb[k]);

  if (!live) return;
  const int nparts = len > 0 ? (len + P_ - 1) / P_ : 1;

  // the two half rows of a row hold the same head over different tokens:
  // add them; the weight sum of head h: its lanes 2 h, 2 h + 1 of both
  // half rows
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i2 = 0; i2 < 16; ++i2) acc[h][i2] += dpp<kDppRor8>(acc[h][i2]);
  float lsum = l_own + dpp<kDppXor1>(l_own);
  lsum += dpp<kDppRor8>(lsum);
  const int64_t q0 = (int64_t)s * a.num_q_heads + g * G;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float L = row_bcast_pair(lsum, h);
    if ((h & 1) != hw) continue;   // the half rows write alternate heads
    float val[16];
#pragma unroll
    for (int i2 = 0; i2 < 16; ++i2) val[i2] = L > 0.f ? acc[h][i2] / L * a.v_scale : 0.f;
    if (nparts == 1) {
      uint4 o0, o1;
      o0.x = pack_bf16x2(val[0], val[1]);
      o0.y = pack_bf16x2(val[2], val[3]);
      o0.z = pack_bf16x2(val[4], val[5]);
      o0.w = pack_bf16x2(val[6], val[7]);
      o1.x = pack_bf16x2(val[8], val[9]);
      o1.y = pack_bf16x2(val[10], val[11]);
      o1.z = pack_bf16x2(val[12], val[13]);
      o1.w = pack_bf16x2(val[14], val[15]);
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (q0 + h) * D + 16 * c);
      dst[0] = o0;
      dst[1] = o1;
    } else {
      float4* dst = reinterpret_cast<float4*>(a.ws_out + ((q0 + h) * a.max_parts + part) * D + 16 * c);
      dst[0] = make_float4(val[0], val[1], val[2], val[3]);
      dst[1] = make_float4(val[4], val[5], val[6], val[7]);
      dst[2] = make_float4(val[8], val[9], val[10], val[11]);
      dst[3] = make_float4(val[12], val[13], val[14], val[15]);
    }
  }
  if (hw == 0 && (c & 1) == 0 && c / 2 < G) {
    const int h = c / 2;
    const float lse2 = lsum > 0.f ? m_own + fast_log2(lsum) : kNegInf;
    if (nparts == 1) {
      if (a.lse) a.lse[q0 + h] = lse2 * kLn2;
    } else {
      a.ws_lse[(q0 + h) * a.max_parts + part] = lse2;
    }
  }
}

}  // namespace decode_body
}  // namespace pa
