// Matrix-matrix kernel (M >= 16): y = x . dequant(Wq)^T (+ bias) on MFMA.
//
// The pages ask whether the decode approach of "metal lowbit kernels:
// qmv_fast optimization" would also work for a GEMM (closing review comment);
// batched int4 weight-only decode on the H100 table of "Add support for fbgemm
// int4 mm kernel" shows why a batched path matters.  Here each K-step of a
// weight tile is dequantized once (w = s*q + z in fp32, rounded to the
// activation type) into LDS and consumed by v_mfma_f32_16x16x32_{f16,bf16}
// with fp32 accumulation.
//
// Tile: 64 (M) x 64 (N) per 256-thread block, K-step 32 (one MFMA deep, and
// never more than one group since every group size is a multiple of 32).
// Wave w computes the 32 x 32 sub-tile (w & 1, w >> 1) as 2 x 2 MFMA tiles.
#include "device_common.h"
#include "kernels.h"

namespace lowbit {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

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

constexpr int QMM_BM = 64, QMM_BN = 64, QMM_BK = 32;
constexpr int QMM_LDS_STRIDE = QMM_BK + 8;   // 16-bit elements per LDS row (pad 16 B)

template <int BITS, int GROUP, int ACT>
__global__ __launch_bounds__(256) void qmm_kernel(QmmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[QMM_BM * QMM_LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[QMM_BN * QMM_LDS_STRIDE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int m_base = blockIdx.y * QMM_BM;
  const int n_base = blockIdx.x * QMM_BN;
  const int wm = (wave & 1) * 32;
  const int wn = (wave >> 1) * 32;

  // staging roles: thread -> (row, 8-element chunk) of the 64 x 32 tiles
  const int st_row = tid >> 2;
  const int st_chunk = tid & 3;
  const int am = m_base + st_row;
  const int bn = n_base + st_row;

  float4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < p.K; k0 += QMM_BK) {
    // ---- activations: 8 elements (16 B) per thread
    uint4 av = make_uint4(0, 0, 0, 0);
    if (am < p.M) {
      av = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) +
                                           static_cast<int64_t>(am) * p.K + k0 + 8 * st_chunk);
    }
    // ---- weights: 8 codes = BITS bytes per thread, dequantized to 16-bit
    uint4 bv = make_uint4(0, 0, 0, 0);
    if (bn < p.N) {
      const uint8_t* src = p.packed + static_cast<int64_t>(bn) * p.row_bytes +
                           ((k0 + 8 * st_chunk) >> 3) * BITS;
      uint64_t stream = 0;
#pragma unroll
      for (int b = 0; b < BITS; ++b) stream |= static_cast<uint64_t>(src[b]) << (8 * b);
      const int64_t gi = static_cast<int64_t>(bn) * p.groups + k0 / GROUP;
      const float s = load_act<ACT>(p.scales, gi);
      const float z = load_act<ACT>(p.zeros, gi);
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = static_cast<float>((stream >> (i * BITS)) & ((1u << BITS) - 1u));
        h[i] = float_to_act_bits<ACT>(__builtin_fmaf(s, q, z));
      }
      bv = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
    }
    *reinterpret_cast<uint4*>(&As[st_row * QMM_LDS_STRIDE + 8 * st_chunk]) = av;
    *reinterpret_cast<uint4*>(&Bs[st_row * QMM_LDS_STRIDE + 8 * st_chunk]) = bv;
    __syncthreads();

    const int fr = lane & 15;        // row within a 16-row MFMA tile
    const int fk = (lane >> 4) * 8;  // first K of this lane's 8 elements
    uint4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = *reinterpret_cast<const uint4*>(&As[(wm + 16 * i + fr) * QMM_LDS_STRIDE + fk]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const uint4*>(&Bs[(wn + 16 * j + fr) * QMM_LDS_STRIDE + fk]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x32<ACT>(a[i], b[j], acc[i][j]);
    __syncthreads();
  }

  // ---- epilogue: lane holds D[4*(lane/16) + r][lane % 16] of each 16x16 tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n_base + wn + 16 * j + (lane & 15);
    if (n >= p.N) continue;
    const float bias = p.bias ? load_act<ACT>(p.bias, n) : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m_base + wm + 16 * i + 4 * (lane >> 4) + r;
        if (m < p.M) store_act<ACT>(p.y, static_cast<int64_t>(m) * p.N + n, acc[i][j][r] + bias);
      }
    }
  }
}

template <int BITS, int GROUP>
static hipError_t dispatch_act(const QmmParams& p, int act, dim3 g, dim3 b, hipStream_t s) {
  switch (act) {
    case ACT_F16: qmm_kernel<BITS, GROUP, ACT_F16><<<g, b, 0, s>>>(p); break;
    case ACT_BF16: qmm_kernel<BITS, GROUP, ACT_BF16><<<g, b, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t dispatch_group(const QmmParams& p, int group, int act, dim3 g, dim3 b,
                                 hipStream_t s) {
  switch (group) {
    case 32: return dispatch_act<BITS, 32>(p, act, g, b, s);
    case 64: return dispatch_act<BITS, 64>(p, act, g, b, s);
    case 128: return dispatch_act<BITS, 128>(p, act, g, b, s);
    case 256: return dispatch_act<BITS, 256>(p, act, g, b, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_qmm(const QmmParams& p, int bits, int group, int act, hipStream_t s) {
  dim3 grid((p.N + QMM_BN - 1) / QMM_BN, (p.M + QMM_BM - 1) / QMM_BM), block(256);
  switch (bits) {
    case 1: return dispatch_group<1>(p, group, act, grid, block, s);
    case 2: return dispatch_group<2>(p, group, act, grid, block, s);
    case 3: return dispatch_group<3>(p, group, act, grid, block, s);
    case 4: return dispatch_group<4>(p, group, act, grid, block, s);
    case 5: return dispatch_group<5>(p, group, act, grid, block, s);
    case 6: return dispatch_group<6>(p, group, act, grid, block, s);
    case 7: return dispatch_group<7>(p, group, act, grid, block, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lowbit
