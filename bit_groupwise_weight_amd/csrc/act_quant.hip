// Dynamic int8 quantization of activation rows, for the activation-quantized
// linear ("[MPS] Add support for Int4 groupwise quantization": the export
// mode with 8-bit dynamic activations and 4-bit weights in groups of 32; the
// page names the mode, the steps below are this library's reading of it).
//
// Per row m, in fp32 with single IEEE operations (compiled without
// contraction):
//   a_m = max_k |x[m, k]| / 127                       (correctly rounded divide)
//   xq[m, k] = clamp(rint_half_even(x[m, k] / a_m), -127, 127)
// a row whose a_m is 0 gets codes 0; a row holding a NaN or an infinity gets
// a_m = NaN and codes 0 (its outputs through the linear are NaN).
//
// One block of 256 threads per row: each thread takes 16-element chunks
// c = tid, tid + 256, ...; the maximum and the non-finite flag are reduced
// across the block, then the chunks are read again (from cache) and written
// as 16 codes in one 16-byte store.
#include "device_common.h"
#include "kernels.h"

namespace lowbit {

constexpr int kActQuantThreads = 256;

// The 16 values of chunk c of a row as fp32 (exact for every input type).
template <int ACT>
__device__ __forceinline__ void load_chunk(const void* row, int c, float (&v)[16]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src = static_cast<const u32x4*>(row);
  if constexpr (ACT == ACT_F32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = src[4 * c + q];
      v[4 * q + 0] = __uint_as_float(w.x);
      v[4 * q + 1] = __uint_as_float(w.y);
      v[4 * q + 2] = __uint_as_float(w.z);
      v[4 * q + 3] = __uint_as_float(w.w);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4 w = src[2 * c + q];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = act_bits_to_float<ACT>(ws[i] & 0xffffu);
        v[8 * q + 2 * i + 1] = act_bits_to_float<ACT>(ws[i] >> 16);
      }
    }
  }
}

template <int ACT>
__global__ __launch_bounds__(kActQuantThreads) void act_quant_i8_kernel(ActQuantParams p) {
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int chunks = p.K / 16;
  const char* row = static_cast<const char*>(p.x) + static_cast<size_t>(m) * p.K * Act<ACT>::bytes;

  float amax = 0.0f;
  bool bad = false;
  for (int c = tid; c < chunks; c += kActQuantThreads) {
    float v[16];
    load_chunk<ACT>(row, c, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = fabsf(v[i]);
      bad |= !(a <= 3.402823466e38f);         // NaN or infinity
      amax = fmaxf(amax, a);
    }
  }
  // block reduction: the maximum of non-negative floats, and the flag
  for (int o = 32; o >= 1; o >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o));
    bad |= __shfl_xor(static_cast<int>(bad), o) != 0;
  }
  __shared__ float s_max[kActQuantThreads / 64];
  __shared__ int s_bad[kActQuantThreads / 64];
  if ((tid & 63) == 0) {
    s_max[tid >> 6] = amax;
    s_bad[tid >> 6] = bad;
  }
  __syncthreads();
  amax = s_max[0];
  bad = s_bad[0] != 0;
#pragma unroll
  for (int w = 1; w < kActQuantThreads / 64; ++w) {
    amax = fmaxf(amax, s_max[w]);
    bad |= s_bad[w] != 0;
  }

  const float a = bad ? __builtin_nanf("") : amax / 127.0f;
  const bool zero = bad || a == 0.0f;
  if (tid == 0) p.ascale[m] = a;

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4* dst = reinterpret_cast<u32x4*>(p.xq + static_cast<size_t>(m) * p.K);
  for (int c = tid; c < chunks; c += kActQuantThreads) {
    uint32_t out[4] = {0u, 0u, 0u, 0u};
    if (!zero) {
      float v[16];
      load_chunk<ACT>(row, c, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t = fminf(fmaxf(__builtin_rintf(v[i] / a), -127.0f), 127.0f);
        out[i >> 2] |= (static_cast<uint32_t>(static_cast<int>(t)) & 0xffu) << (8 * (i & 3));
      }
    }
    dst[c] = u32x4{out[0], out[1], out[2], out[3]};
  }
}

hipError_t launch_act_quant_i8(const ActQuantParams& p, int act, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.M)), block(kActQuantThreads);
  switch (act) {
    case ACT_F32: act_quant_i8_kernel<ACT_F32><<<grid, block, 0, stream>>>(p); break;
    case ACT_F16: act_quant_i8_kernel<ACT_F16><<<grid, block, 0, stream>>>(p); break;
    default: act_quant_i8_kernel<ACT_BF16><<<grid, block, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace lowbit
