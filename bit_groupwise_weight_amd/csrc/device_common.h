// Device-side helpers shared by the HIP kernels of the low-bit linear layer.
// gfx950 (CDNA4) only: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kernels.h"

namespace lowbit {

template <int ACT> struct Act;
template <> struct Act<ACT_F32> { using bits_t = uint32_t; static constexpr int bytes = 4; };
template <> struct Act<ACT_F16> { using bits_t = uint16_t; static constexpr int bytes = 2; };
template <> struct Act<ACT_BF16> { using bits_t = uint16_t; static constexpr int bytes = 2; };

// ---- element conversions (all exact or round-to-nearest-even) -------------

__device__ __forceinline__ float f16_bits_to_float(uint32_t b) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(b)));
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}
template <int ACT> __device__ __forceinline__ float act_bits_to_float(uint32_t b) {
  if constexpr (ACT == ACT_F32) return __uint_as_float(b);
  else if constexpr (ACT == ACT_F16) return f16_bits_to_float(b);
  else return bf16_bits_to_float(b);
}

// fp32 -> bf16, nearest even (inputs here are finite or +-inf; NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t float_to_f16_bits(float f) {
  return __half_as_ushort(__float2half_rn(f));
}
template <int ACT> __device__ __forceinline__ uint32_t float_to_act_bits(float f) {
  if constexpr (ACT == ACT_F32) return __float_as_uint(f);
  else if constexpr (ACT == ACT_F16) return float_to_f16_bits(f);
  else return float_to_bf16_bits(f);
}

template <int ACT>
__device__ __forceinline__ float load_act(const void* base, size_t idx) {
  using T = typename Act<ACT>::bits_t;
  return act_bits_to_float<ACT>(static_cast<const T*>(base)[idx]);
}
template <int ACT>
__device__ __forceinline__ void store_act(void* base, size_t idx, float v) {
  using T = typename Act<ACT>::bits_t;
  static_cast<T*>(base)[idx] = static_cast<T>(float_to_act_bits<ACT>(v));
}

// ---- packed-code extraction ------------------------------------------------
// A run of 32 consecutive codes of width BITS occupies exactly BITS 32-bit
// words (LSB-first stream).  Code I (0..31) starts at stream bit I*BITS.
template <int BITS, int I>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w) {
  constexpr int p = I * BITS;
  constexpr int d = p >> 5;
  constexpr int o = p & 31;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if constexpr (o + BITS <= 32) {
    return (w[d] >> o) & mask;
  } else {
    return __builtin_amdgcn_alignbit(w[d + 1], w[d], o) & mask;
  }
}

// ---- dot products ----------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi with fp32 accumulation; a, b hold two 16-bit
// values of the activation type.
template <int ACT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (ACT == ACT_F16) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  acc, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), acc, false);
  }
}

// Two ones of the activation type in one word: dot2 with it sums a pair.
template <int ACT> struct Magic;
template <> struct Magic<ACT_F16> { static constexpr uint32_t ones = 0x3c003c00u; };
template <> struct Magic<ACT_BF16> { static constexpr uint32_t ones = 0x3f803f80u; };

// ---- cross-lane sums with DPP ----------------------------------------------
// x + (x moved by a DPP pattern); lanes outside row_mask add 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_add(float x) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
  return x + __int_as_float(moved);
}

// Sum over aligned groups of `lanes` lanes (1, 2, ..., 64; uniform).  The
// group's total ends up in its LAST lane (lane % lanes == lanes - 1).
__device__ __forceinline__ float group_sum_to_last(float x, int lanes) {
  if (lanes >= 2) x = dpp_add<0xb1>(x);          // quad_perm [1,0,3,2]
  if (lanes >= 4) x = dpp_add<0x4e>(x);          // quad_perm [2,3,0,1]
  if (lanes >= 8) x = dpp_add<0x141>(x);         // row_half_mirror
  if (lanes >= 16) x = dpp_add<0x140>(x);        // row_mirror
  if (lanes >= 32) x = dpp_add<0x142, 0xa>(x);   // row_bcast15 into rows 1 and 3
  if (lanes >= 64) x = dpp_add<0x143, 0x8>(x);   // row_bcast31 into row 3
  return x;
}

}  // namespace lowbit
