// Quantize + pack kernel: weights (fp32, or fp16 / bf16 upcast exactly to
// fp32) -> per-(row, group) scale and zero,
// unsigned b-bit codes and the LSB-first contiguous packed stream.
//
// Format (pages "Add torchao mps ops", linear:afpwx description, and
// "metal lowbit kernels: qmv_fast optimization", Summary): groups of `group`
// consecutive K-elements of a row share one scale and one zero, stored
// N x num_groups; codes are stored back to back across byte boundaries.
//
// Arithmetic, all fp32 single operations in this order (compiled with
// -ffp-contract=off, correctly rounded divide):
//   mn, mx = min, max over the group (a zero result is taken as +0)
//   s = (mx - mn) / (2^b - 1);  z = mn
//   s_st, z_st = s, z rounded to the storage dtype (nearest even)
//   q = s_st == 0 ? 0 : clamp(rint_half_even((w - z_st) / s_st), 0, 2^b - 1)
//
// Work decomposition: one thread per 8-code atom (8 consecutive K-elements,
// which pack into exactly `bits` bytes).  The group/8 threads of a group are
// consecutive lanes of one wavefront and combine min/max with lane shuffles.
#include "device_common.h"
#include "kernels.h"

namespace lowbit {

// The 8 weights of one atom as fp32 (fp16 and bf16 values are exact in fp32).
template <int W_ACT>
__device__ __forceinline__ void load_atom(const void* w, int64_t off, float (&out)[8]) {
  if constexpr (W_ACT == ACT_F32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(w) + off);
    const float4 v0 = src[0], v1 = src[1];
    out[0] = v0.x; out[1] = v0.y; out[2] = v0.z; out[3] = v0.w;
    out[4] = v1.x; out[5] = v1.y; out[6] = v1.z; out[7] = v1.w;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + off);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = act_bits_to_float<W_ACT>(d[i] & 0xFFFFu);
      out[2 * i + 1] = act_bits_to_float<W_ACT>(d[i] >> 16);
    }
  }
}

template <int SZ_ACT, int W_ACT>
__global__ __launch_bounds__(256) void quant_pack_kernel(QuantParams p) {
  const int64_t atoms_per_row = p.K >> 3;
  const int64_t total = p.N * atoms_per_row;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool valid = t < total;           // whole groups are either valid or not
  const int64_t tt = valid ? t : 0;
  const int64_t n = tt / atoms_per_row;
  const int64_t a = tt - n * atoms_per_row;
  const int seg = p.group >> 3;           // threads per group: 4, 8, 16 or 32

  float w[8];
  load_atom<W_ACT>(p.w, n * p.K + a * 8, w);
  bool finite = true;
  float mn = w[0], mx = w[0];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    finite = finite && (__builtin_fabsf(w[i]) <= 3.402823466e38f);
    mn = w[i] < mn ? w[i] : mn;
    mx = w[i] > mx ? w[i] : mx;
  }
  for (int off = seg >> 1; off > 0; off >>= 1) {
    float omn = __shfl_xor(mn, off);
    float omx = __shfl_xor(mx, off);
    mn = omn < mn ? omn : mn;
    mx = omx > mx ? omx : mx;
  }
  if (valid && !finite) p.status[0] = 1;
  if (mn == 0.0f) mn = 0.0f;   // canonical +0
  if (mx == 0.0f) mx = 0.0f;

  const float qmax = static_cast<float>((1 << p.bits) - 1);
  const float s32 = (mx - mn) / qmax;
  const uint32_t s_bits = float_to_act_bits<SZ_ACT>(s32);
  const uint32_t z_bits = float_to_act_bits<SZ_ACT>(mn);
  const float s_st = act_bits_to_float<SZ_ACT>(s_bits);
  const float z_st = act_bits_to_float<SZ_ACT>(z_bits);
  const bool sz_finite = (__builtin_fabsf(s_st) <= 3.402823466e38f) &&
                         (__builtin_fabsf(z_st) <= 3.402823466e38f);

  const int64_t groups = p.K / p.group;
  const int64_t g = (a * 8) / p.group;
  if (valid && (a & (seg - 1)) == 0) {
    using T = typename Act<SZ_ACT>::bits_t;
    static_cast<T*>(p.scales)[n * groups + g] = static_cast<T>(s_bits);
    static_cast<T*>(p.zeros)[n * groups + g] = static_cast<T>(z_bits);
    if (!sz_finite) p.status[1] = 1;
  }

  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t c = 0;
    if (s_st != 0.0f) {
      float tq = (w[i] - z_st) / s_st;
      tq = __builtin_rintf(tq);
      tq = tq < 0.0f ? 0.0f : tq;
      tq = tq > qmax ? qmax : tq;
      c = static_cast<uint32_t>(tq);
    }
    q[i] = c;
  }
  if (!valid) return;

  uint64_t stream = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) stream |= static_cast<uint64_t>(q[i]) << (i * p.bits);
  uint8_t* dst = p.packed + n * ((p.K * p.bits) >> 3) + a * p.bits;
  for (int b = 0; b < p.bits; ++b) dst[b] = static_cast<uint8_t>(stream >> (8 * b));
  if (p.codes != nullptr) {
    uint8_t* c = p.codes + n * p.K + a * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = static_cast<uint8_t>(q[i]);
  }
}

hipError_t launch_quant_pack(const QuantParams& p, hipStream_t stream) {
  const int64_t total = p.N * (p.K >> 3);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks)), block(threads);
  if (p.sz_act < ACT_F32 || p.sz_act > ACT_BF16) return hipErrorInvalidValue;
  switch (p.w_act * 3 + p.sz_act) {
    case ACT_F32 * 3 + ACT_F32: quant_pack_kernel<ACT_F32, ACT_F32><<<grid, block, 0, stream>>>(p); break;
    case ACT_F32 * 3 + ACT_F16: quant_pack_kernel<ACT_F16, ACT_F32><<<grid, block, 0, stream>>>(p); break;
    case ACT_F32 * 3 + ACT_BF16: quant_pack_kernel<ACT_BF16, ACT_F32><<<grid, block, 0, stream>>>(p); break;
    case ACT_F16 * 3 + ACT_F32: quant_pack_kernel<ACT_F32, ACT_F16><<<grid, block, 0, stream>>>(p); break;
    case ACT_F16 * 3 + ACT_F16: quant_pack_kernel<ACT_F16, ACT_F16><<<grid, block, 0, stream>>>(p); break;
    case ACT_F16 * 3 + ACT_BF16: quant_pack_kernel<ACT_BF16, ACT_F16><<<grid, block, 0, stream>>>(p); break;
    case ACT_BF16 * 3 + ACT_F32: quant_pack_kernel<ACT_F32, ACT_BF16><<<grid, block, 0, stream>>>(p); break;
    case ACT_BF16 * 3 + ACT_F16: quant_pack_kernel<ACT_F16, ACT_BF16><<<grid, block, 0, stream>>>(p); break;
    case ACT_BF16 * 3 + ACT_BF16: quant_pack_kernel<ACT_BF16, ACT_BF16><<<grid, block, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lowbit
