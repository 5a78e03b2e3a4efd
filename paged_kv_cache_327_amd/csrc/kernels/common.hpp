// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// fp32 c + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Two floats rounded to nearest-even bf16 and packed (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Sum over each aligned group of 8 lanes (all 8 receive the total):
// xor-1 and xor-2 quad permutes, then the half-row mirror (lane i <-> 7 - i).
__device__ __forceinline__ float sum_lanes8(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
  return x;
}

// Cross-lane moves within rows of 16 lanes (DPP): quad permutes, the
// half-row mirror (lane i <-> 7 - i) and the row rotation by 8.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppBcast0 = 0x00;      // quad_perm [0, 0, 0, 0]
constexpr int kDppBcast2 = 0xAA;      // quad_perm [2, 2, 2, 2]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;  // lane i <-> 15 - i
constexpr int kDppRowBcast0 = 0x150;  // + n: lane n of each 16-lane row to the whole row
constexpr int kDppRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// E4M3 (finite-only form: bias 7, subnormals m * 2^-9, largest finite 448,
// S.1111.111 = NaN) code of an fp32 value: round to nearest, ties to even;
// magnitudes above 448 and infinities saturate to 448; NaN gives the NaN code.
// Written from the format's definition with integer operations, so the result
// does not depend on a conversion instruction's rounding or clamping mode.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7fffffffu;
  uint32_t code;
  if (mag > 0x7f800000u) {
    code = 0x7fu;                                   // NaN
  } else if (mag >= 0x43e00000u) {
    code = 0x7eu;                                   // >= 448: saturate
  } else if (mag < 0x3c800000u) {
    // below 2^-6: a multiple of 2^-9 (code 8, the smallest normal, on carry);
    // scaling by 2^9 is exact and rint rounds half to even
    code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  } else {
    // keep 3 of the 23 mantissa bits, round to nearest even on the other 20;
    // a carry moves into the exponent; rebias 127 -> 7
    const uint32_t r = mag + 0x7ffffu + ((mag >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
    code = code > 0x7eu ? 0x7eu : code;
  }
  return code | sign;
}

// Two E4M3 codes (bytes 0-1 of w, or bytes 2-3 with HI) as a packed bf16 pair
// (lo = the lower byte).  Exact: every E4M3 value is a bf16 value, and the
// scale operand is 1.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pa
