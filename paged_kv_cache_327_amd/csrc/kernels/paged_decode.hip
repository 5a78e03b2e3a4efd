// Paged decode attention for gfx950: a split-K partition pass plus a
// log-sum-exp merge.
//
// What is computed ("PagedAttention: fragmentation, blocks, block tables",
// attention-metadata section; "The pantry of pigeonholes", "The mechanism"):
// for sequence s, the kernel walks row s of the block table in logical order
// for ceil(seq_lens[s] / B) entries and attends one query per head over the
// gathered K/V.  The split into partitions is named on the first page
// ("the tiling, the split-K, the paged gather") without detail; the design
// below is ours.
//
// Partition pass: one work-group (4 waves) per (partition, KV head g, seq s).
//  * The partition's block-table entries are staged once in LDS (clamped into
//    [0, num_blocks)), so a token's physical row costs one LDS read.
//  * Lanes form groups of 8.  A group owns one token at a time; its 8 lanes
//    split head_dim into 16-byte pieces (lane i holds d = 8i..8i+7 and, for
//    D = 128, d = 64+8i..64+8i+7), so every K/V row load is a coalesced
//    16-byte-per-lane access of the token's contiguous row.
//  * The G = Hq/Hkv query heads of KV head g are all computed from the same
//    K/V registers (the GQA sharing): q.k with v_dot2_f32_bf16, summed over the
//    8 lanes with DPP; softmax weights are rounded to bf16 and multiplied into
//    V with v_dot2_f32_bf16 on token pairs, accumulating in fp32.
//  * A wave handles 16-token tiles (2 tokens per group) and keeps the next
//    two tiles' K/V loads in flight while it computes the current one.
//  * Online softmax in the log2 domain; the running maximum is only raised
//    when a logit exceeds it by more than 8 (weights stay <= 2^8), which keeps
//    the result exact and makes rescales rare.
//  * Groups and waves are merged with the log-sum-exp identity.  A sequence
//    with one partition writes its bf16 output directly; otherwise partials
//    (normalised output, log2 lse) go to the workspace for the merge pass.
#include "../internal.hpp"
#include "common.hpp"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 16;     // tokens per wave iteration
constexpr int kChunk = 512;   // tokens whose table entries are staged at once
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D>
struct KV {
  static constexpr int kPieces = D / 64;  // 16-byte pieces per lane per token
  uint4 k[2][kPieces];
  uint4 v[2][kPieces];
};

template <int D, int G>
__global__ void __launch_bounds__(256) decode_partition_kernel(DecodeArgs a) {
  constexpr int PPL = D / 64;
  __shared__ int32_t s_bt[kChunk];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];

  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (SGPR) so that the tile loop below branches on scalars
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 3, li = lane & 7;

  int len = a.seq_lens[s];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const int P = a.partition_size;
  const int nparts = len > 0 ? (len + P - 1) / P : 1;
  if (part >= nparts) return;
  const int start = part * P;
  const int end = start + P < len ? start + P : len;
  const int lgB = a.log2_block_size;
  const int Bmask = (1 << lgB) - 1;
  const int64_t row_elems = (int64_t)a.num_kv_heads * D;
  const int64_t bstride = a.cache_block_stride;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.key_cache) + (int64_t)g * D + 8 * li;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.value_cache) + (int64_t)g * D + 8 * li;
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.bt_stride;
  const float scale = a.scale * kLog2e;

  uint4 qr[G][PPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < PPL; ++k)
      qr[h][k] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                 ((int64_t)s * a.num_q_heads + g * G + h) * D + 64 * k + 8 * li);

  float m[G], l[G], acc[G][PPL][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < PPL; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][k][i] = 0.f;
  }

  for (int c0 = start; c0 < end; c0 += kChunk) {
    const int c1 = c0 + kChunk < end ? c0 + kChunk : end;
    const int j0 = c0 >> lgB;
    const int nj = ((c1 - 1) >> lgB) - j0 + 1;
    __syncthreads();
    for (int i = tid; i < nj; i += 256) {
      int b = bt_row[j0 + i];
      b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
      s_bt[i] = b;
    }
    __syncthreads();

    // Tokens past c1 are redirected to token c0 (always valid), so every
    // load stays inside the cache and can be issued unconditionally: with no
    // branch around the prefetches the compiler's wait counts stay exact and
    // the next tiles' loads remain in flight while this one is computed.
    // All K loads are issued before the V loads so q.k can start first.
    auto load = [&](int t0, KV<D>& r) {
      int64_t off[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        int t = t0 + grp + 8 * u;
        t = t < c1 ? t : c0;
        const int64_t blk = s_bt[(t >> lgB) - j0];
        off[u] = blk * bstride + (int64_t)(t & Bmask) * row_elems;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int k = 0; k < PPL; ++k) r.k[u][k] = *reinterpret_cast<const uint4*>(kbase + off[u] + 64 * k);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int k = 0; k < PPL; ++k) r.v[u][k] = *reinterpret_cast<const uint4*>(vbase + off[u] + 64 * k);
    };

    auto compute = [&](int t0, const KV<D>& r) {
      const bool valid0 = t0 + grp < c1;
      const bool valid1 = t0 + grp + 8 < c1;
      float x[G][2];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float d = 0.f;
#pragma unroll
          for (int k = 0; k < PPL; ++k) {
            const uint32_t* qq = reinterpret_cast<const uint32_t*>(&qr[h][k]);
            const uint32_t* kk = reinterpret_cast<const uint32_t*>(&r.k[u][k]);
#pragma unroll
            for (int i = 0; i < 4; ++i) d = dot2_bf16(qq[i], kk[i], d);
          }
          x[h][u] = sum_lanes8(d) * scale;
        }
      uint32_t pp[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float x0 = valid0 ? x[h][0] : kNegInf;
        const float x1 = valid1 ? x[h][1] : kNegInf;
        const float mx = fmaxf(x0, x1);
        if (mx > m[h] + kRescaleSlack) {
          const float alpha = fast_exp2(m[h] - mx);
          l[h] *= alpha;
#pragma unroll
          for (int k = 0; k < PPL; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[h][k][i] *= alpha;
          m[h] = mx;
        }
        const float p0 = valid0 ? fast_exp2(x0 - m[h]) : 0.f;
        const float p1 = valid1 ? fast_exp2(x1 - m[h]) : 0.f;
        pp[h] = pack_bf16x2(p0, p1);
        l[h] += bf16_lo(pp[h]) + bf16_hi(pp[h]);
      }
      // V rows of the two tokens interleaved per d: (v0[d], v1[d]) pairs.
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&r.v[0][k]);
        const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&r.v[1][k]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = __builtin_amdgcn_perm(v1[i], v0[i], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(v1[i], v0[i], 0x07060302u);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][k][2 * i] = dot2_bf16(pp[h], lo, acc[h][k][2 * i]);
            acc[h][k][2 * i + 1] = dot2_bf16(pp[h], hi, acc[h][k][2 * i + 1]);
          }
        }
      }
    };

    // Three register buffers: while tile t is computed, tiles t + 64 and
    // t + 128 are in flight.  The loop runs whole triples and has a single,
    // bottom-tested exit (an exit in the middle gives the compiler a path
    // back into the loop with loads pending, and it then drains every load
    // at the top); the last 0-2 tiles are computed after it from buffers
    // already loaded.  All branches here are wave-uniform.
    constexpr int kStep = kWaves * kTile;
    int t = c0 + wave * kTile;
    const int n_tiles = t < c1 ? (c1 - t + kStep - 1) / kStep : 0;
    if (n_tiles > 0) {
      KV<D> r0, r1, r2;
      load(t, r0);
      load(t + kStep, r1);
      int i = 0;
      for (; i + 3 <= n_tiles; i += 3) {
        load(t + 2 * kStep, r2);
        compute(t, r0);
        t += kStep;
        load(t + 2 * kStep, r0);
        compute(t, r1);
        t += kStep;
        load(t + 2 * kStep, r1);
        compute(t, r2);
        t += kStep;
      }
      if (n_tiles - i >= 1) compute(t, r0);
      if (n_tiles - i >= 2) compute(t + kStep, r1);
    }
  }

  // Merge the 8 lane groups of the wave (butterfly over lanes 8, 16, 32 apart).
#pragma unroll
  for (int sh = 8; sh < 64; sh <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], sh);
      const float lo = __shfl_xor(l[h], sh);
      const float M = fmaxf(m[h], mo);
      const float wa = m[h] == kNegInf ? 0.f : fast_exp2(m[h] - M);
      const float wb = mo == kNegInf ? 0.f : fast_exp2(mo - M);
      l[h] = l[h] * wa + lo * wb;
#pragma unroll
      for (int k = 0; k < PPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][k][i] = acc[h][k][i] * wa + __shfl_xor(acc[h][k][i], sh) * wb;
      m[h] = M;
    }
  }
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int k = 0; k < PPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) s_acc[wave][h][64 * k + 8 * li + i] = acc[h][k][i];
      if (lane == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves: thread -> (head h, dim d) outputs.
  for (int o = tid; o < G * D; o += 256) {
    const int h = o / D, d = o % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = s_m[w][h];
        const float e = mw == kNegInf ? 0.f : fast_exp2(mw - M);
        L += s_l[w][h] * e;
        A += s_acc[w][h][d] * e;
      }
    }
    const int hq = g * G + h;
    const int64_t row = (int64_t)s * a.num_q_heads + hq;
    const float val = L > 0.f ? A / L : 0.f;
    const float lse2 = L > 0.f ? M + fast_log2(L) : kNegInf;
    if (nparts == 1) {
      static_cast<uint16_t*>(a.out)[row * D + d] = to_bf16(val);
      if (a.lse && d == 0) a.lse[row] = lse2 * kLn2;
    } else {
      a.ws_out[(row * a.max_parts + part) * D + d] = val;
      if (d == 0) a.ws_lse[row * a.max_parts + part] = lse2;
    }
  }
}

// out[s, h] = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M) over the
// sequence's partitions (log-sum-exp identity); lse = (M + log2 W) ln 2.
template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  int len = a.seq_lens[s];
  len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
  const int nparts = (len + a.partition_size - 1) / a.partition_size;
  if (nparts <= 1) return;
  const int64_t row = (int64_t)s * a.num_q_heads + hq;
  const float* lse2 = a.ws_lse + row * a.max_parts;
  const float* po = a.ws_out + row * a.max_parts * D;
  float M = kNegInf;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, lse2[p]);
  float W = 0.f, o[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(lse2[p] - M);
    W += w;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) o[i] += w * po[p * D + lane + 64 * i];
  }
#pragma unroll
  for (int i = 0; i < D / 64; ++i) static_cast<uint16_t*>(a.out)[row * D + lane + 64 * i] = to_bf16(o[i] / W);
  if (a.lse && lane == 0) a.lse[row] = (M + fast_log2(W)) * kLn2;
}

template <int D, int G>
int launch_g(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_partition_kernel<D, G>), dim3(a.max_parts, a.num_kv_heads, a.num_seqs), dim3(256), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return (int)e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0, st, a);
  return (int)hipGetLastError();
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

}  // namespace

int launch_paged_decode(const DecodeArgs& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace pa
