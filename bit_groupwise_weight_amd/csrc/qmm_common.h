// Pieces shared by the two MFMA kernels (fp16 and bf16 activations):
// operand types, the K step, code-run loads and the activation stage layout.
#pragma once

#include <utility>

#include "device_common.h"
#include "kernels.h"

namespace lowbit {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v_t __attribute__((ext_vector_type(2)));

template <int ACT>
__device__ __forceinline__ float4_t mfma16x16x32(uint4 a, uint4 b, float4_t c) {
  if constexpr (ACT == ACT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                   __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
  }
}

// Two fp32 values -> two activation-type values (nearest even), packed.
template <int ACT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const float2_t v = {lo, hi};
  if constexpr (ACT == ACT_F16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2v_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf162v_t));
  }
}

constexpr int QMM_BK = 128;    // K per step

// The BITS words of one 32-code run (4-byte aligned) in one vector load for
// BITS <= 4 and two above.
template <int BITS>
__device__ __forceinline__ void load_run_words(const uint8_t* src, uint32_t (&w)[BITS]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const uint8_t* s = static_cast<const uint8_t*>(__builtin_assume_aligned(src, 4));
  constexpr int O = BITS >= 4 ? 4 : 0;
  constexpr int REST = BITS - O;
  if constexpr (BITS >= 4) {
    u32x4 v;
    __builtin_memcpy(&v, s, 16);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  if constexpr (REST == 3) {
    u32x3 v;
    __builtin_memcpy(&v, s + 4 * O, 12);
    w[O] = v.x; w[O + 1] = v.y; w[O + 2] = v.z;
  } else if constexpr (REST == 2) {
    u32x2 v;
    __builtin_memcpy(&v, s + 4 * O, 8);
    w[O] = v.x; w[O + 1] = v.y;
  } else if constexpr (REST == 1) {
    __builtin_memcpy(&w[O], s + 4 * O, 4);
  }
}

// a & 0x0f0f0f0f, opaque to the optimizer (which would otherwise fold the
// masking into one bit-field extract per code and lose the byte planes)
__device__ __forceinline__ uint32_t and_nibbles(uint32_t a) {
  uint32_t r;
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(r) : "v"(a));
  return r;
}

template <int I>
__device__ __forceinline__ float ubyte(uint32_t v) {  // v_cvt_f32_ubyte<I>
  return static_cast<float>((v >> (8 * I)) & 0xFFu);
}

// LDS swizzle of the activation stage: chunk c of row r sits at position
// c ^ stage_swizzle(r & 15), the 4-bit row index rotated by two bits.  A
// k-sub read of an MFMA tile (16 rows, 4 lane groups of 16 lanes) then runs at
// ~200 B/clk per CU on gfx950; the plain c ^ (r & 15) measured 120 B/clk
// (contiguous reads: 234).
__device__ __forceinline__ int stage_swizzle(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

}  // namespace lowbit
