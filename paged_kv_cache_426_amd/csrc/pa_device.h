// Device helpers shared by the gfx950 kernels: element conversions, 16-lane
// and 64-lane reductions on DPP, and the E4M3FN encoder of the slot write.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

template <int DT> struct ElemBytes;
template <> struct ElemBytes<PA_F32> { static constexpr int value = 4; };
template <> struct ElemBytes<PA_F16> { static constexpr int value = 2; };
template <> struct ElemBytes<PA_BF16> { static constexpr int value = 2; };
template <> struct ElemBytes<PA_FP8_E4M3FN> { static constexpr int value = 1; };
template <> struct ElemBytes<PA_INT8> { static constexpr int value = 1; };

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------

// The two bfloat16 halves of a word, widened exactly (a bfloat16 is the top
// half of a binary32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).x;
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).y;
}

// float32 -> bfloat16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// float32 -> OCP E4M3FN, round to nearest even, saturate to +-448, NaN ->
// 0x7F | sign. Integer formulation on the binary32 fields:
//  * |x| >= 448 saturates (the largest code is exponent 15, mantissa 6);
//  * |x| >= 2^-6 (binary32 biased exponent >= 121) is an E4M3FN normal:
//    keep the top 3 of the 23 mantissa bits with round-half-even on bit 20,
//    then rebias the exponent from 127 to 7 (a mantissa carry moves into
//    the exponent field by itself);
//  * below 2^-6 the code is the number of 2^-9 steps, rounded half-even;
//    8 steps is the smallest normal, whose code is also 8.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float f) {
  const uint32_t u = f2u(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // 448.0f
  const uint32_t e = a >> 23;
  if (e >= 121u) {
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
  }
  if (e == 0u) return sign;  // binary32 zero or subnormal: far below 2^-10
  // |x| = m * 2^(e-150) with the implicit bit; in units of 2^-9 that is
  // m * 2^(e-141), a right shift by s = 141 - e >= 21.
  const uint32_t m = (a & 0x7fffffu) | 0x800000u;
  const uint32_t s = 141u - e;
  if (s > 25u) return sign;  // below 2^-11: rounds to zero
  const uint32_t q = (m + (1u << (s - 1u)) - 1u + ((m >> s) & 1u)) >> s;
  return sign | q;
}

// float32 -> symmetric int8 code (low byte of the result): round to
// nearest, ties to even (v_rndne), saturating to [-127, 127]; NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_int8(float f) {
  if (f != f) return 0u;
  const float r = fminf(fmaxf(__builtin_rintf(f), -127.0f), 127.0f);
  return (uint32_t)(int32_t)r & 0xffu;
}

// ---------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------

// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror (lane i of
// each 8 reads lane 7-i), row_mirror (lane i of each 16 reads lane 15-i).
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xf, 0xf, true);
}

// Sum over aligned groups of N lanes (N a power of two, 1..64); every lane of
// a group gets the same bits (each step adds two equal partial sums in
// swapped order, and float addition is commutative).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Integer sum over aligned groups of N lanes.
template <int N>
__device__ __forceinline__ int group_sum_i(int v) {
#pragma unroll
  for (int off = 1; off < N; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

}  // namespace pa
