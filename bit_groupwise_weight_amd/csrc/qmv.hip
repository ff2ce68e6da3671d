// Decode matrix-vector kernel (small M): y = x . dequant(Wq)^T (+ bias).
//
// Prior art: the qmv_fast Metal kernel of "metal lowbit kernels: qmv_fast
// optimization" (Summary) streams packed rows and applies the N x num_groups
// scales and zeros in the inner loop.  This kernel keeps that idea and is laid
// out for CDNA4:
//   * a row's codes are cut into 128-code units; a unit of b-bit codes is
//     exactly b x 16 bytes, fetched with b 128-bit loads;
//   * 2^lpr_shift lanes of one wavefront share a group of R rows, each lane
//     walking units u = lane, lane + lanes, ...; the lane holds the activation
//     slice of its unit in registers and reuses it for all R rows;
//   * codes are unpacked in registers; for fp16/bf16 activations two codes are
//     OR-ed into the mantissas of a 16-bit pair (value MAGIC + q, exact) and
//     multiplied into an fp32 accumulator with one dot2 instruction; the MAGIC
//     offset is removed per 32-code run with the run's activation sum X:
//       sum x*q = P - MAGIC * X
//   * per 32-code run (which never crosses a group): y += s*(sum x*q) + z*X,
//     i.e. sum_k x_k (s q_k + z) without forming the dequantized weight;
//   * partial sums of the lanes of a row group are combined with lane
//     shuffles, then bias is added in fp32 and the result rounded once.
#include "device_common.h"
#include "kernels.h"

#ifndef LOWBIT_BITS
#error "compile with -DLOWBIT_BITS=<1..7>"
#endif

namespace lowbit {

// Load the 16*BITS bytes of one 128-code unit of one row (or the leading
// nsub 32-code runs of a ragged last unit) into 4*BITS words.
template <int BITS>
__device__ __forceinline__ void load_unit(const uint8_t* rowp, bool vec16, int nsub,
                                          uint32_t (&d)[4 * BITS]) {
  if (vec16) {
    const uint4* s = reinterpret_cast<const uint4*>(rowp);
#pragma unroll
    for (int i = 0; i < BITS; ++i) {
      uint4 v = s[i];
      d[4 * i + 0] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
    }
  } else {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(rowp);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < BITS; ++i) d[j * BITS + i] = (j < nsub) ? s[j * BITS + i] : 0u;
    }
  }
}

// sum over 32 codes of x_k * (MAGIC + q_k), x given as 16 packed pairs.
template <int BITS, int ACT, int I = 0>
__device__ __forceinline__ float dot_run_pairs(const uint32_t* w, const uint32_t* xp, float acc) {
  if constexpr (I < 16) {
    const uint32_t c0 = code_at<BITS, 2 * I>(w);
    const uint32_t c1 = code_at<BITS, 2 * I + 1>(w);
    const uint32_t h = c0 | (c1 << 16) | Magic<ACT>::pair;
    acc = dot2<ACT>(xp[I], h, acc);
    return dot_run_pairs<BITS, ACT, I + 1>(w, xp, acc);
  } else {
    return acc;
  }
}

// sum over 32 codes of x_k * q_k, x as fp32.
template <int BITS, int I = 0>
__device__ __forceinline__ float dot_run_f32(const uint32_t* w, const float* xf, float acc) {
  if constexpr (I < 32) {
    const float q = static_cast<float>(code_at<BITS, I>(w));
    acc = __builtin_fmaf(xf[I], q, acc);
    return dot_run_f32<BITS, I + 1>(w, xf, acc);
  } else {
    return acc;
  }
}

template <int BITS, int GROUP, int ACT, int MT>
__global__ __launch_bounds__(256) void qmv_kernel(QmvParams p) {
  constexpr int R = (MT == 1) ? 2 : 1;          // rows per row group
  constexpr int XW = (ACT == ACT_F32) ? 32 : 16; // words of x per 32-code run
  const int tid = threadIdx.x;
  const int lanes = 1 << p.lpr_shift;
  const int lane = tid & (lanes - 1);
  const int rg = tid >> p.lpr_shift;
  const int rgs = blockDim.x >> p.lpr_shift;
  const int n_base = (blockIdx.x * rgs + rg) * R;
  const int m0 = blockIdx.y * MT;

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  for (int u = lane; u < p.units; u += lanes) {
    const int k0 = u * 128;
    const int nsub = min(4, (p.K - k0) >> 5);
    const bool vec16 = p.aligned16 && nsub == 4;

    uint32_t d[R][4 * BITS];
    float sv[R][4], zv[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n_base + r;
      if (n < p.N) {
        load_unit<BITS>(p.packed + static_cast<int64_t>(n) * p.row_bytes +
                            static_cast<int64_t>(u) * 16 * BITS,
                        vec16, nsub, d[r]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int g = min((k0 + 32 * j) / GROUP, p.groups - 1);
          const int64_t gi = static_cast<int64_t>(n) * p.groups + g;
          sv[r][j] = load_act<ACT>(p.scales, gi);
          zv[r][j] = load_act<ACT>(p.zeros, gi);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4 * BITS; ++i) d[r][i] = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) { sv[r][j] = 0.0f; zv[r][j] = 0.0f; }
      }
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= nsub) break;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m0 + m >= p.M) break;
        const uint8_t* xrow = static_cast<const uint8_t*>(p.x) +
                              (static_cast<int64_t>(m0 + m) * p.K + k0 + 32 * j) * Act<ACT>::bytes;
        uint32_t xw[XW];
        const uint4* xs = reinterpret_cast<const uint4*>(xrow);
#pragma unroll
        for (int i = 0; i < XW / 4; ++i) {
          uint4 v = xs[i];
          xw[4 * i + 0] = v.x; xw[4 * i + 1] = v.y; xw[4 * i + 2] = v.z; xw[4 * i + 3] = v.w;
        }
        float X = 0.0f;
        if constexpr (ACT == ACT_F32) {
#pragma unroll
          for (int i = 0; i < 32; ++i) X += __uint_as_float(xw[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) X = dot2<ACT>(xw[i], Magic<ACT>::ones, X);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float dotq;
          if constexpr (ACT == ACT_F32) {
            dotq = dot_run_f32<BITS>(&d[r][j * BITS], reinterpret_cast<const float*>(xw), 0.0f);
          } else {
            const float P = dot_run_pairs<BITS, ACT>(&d[r][j * BITS], xw, 0.0f);
            dotq = P - Magic<ACT>::value * X;
          }
          acc[r][m] = __builtin_fmaf(sv[r][j], dotq, acc[r][m]);
          acc[r][m] = __builtin_fmaf(zv[r][j], X, acc[r][m]);
        }
      }
    }
  }

  // combine the partial sums of the row group's lanes (stays inside the
  // aligned group of `lanes` lanes of this wavefront)
  for (int off = lanes >> 1; off > 0; off >>= 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] += __shfl_xor(acc[r][m], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n_base + r;
      if (n >= p.N) continue;
      const float b = p.bias ? load_act<ACT>(p.bias, n) : 0.0f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m0 + m >= p.M) break;
        store_act<ACT>(p.y, static_cast<int64_t>(m0 + m) * p.N + n, acc[r][m] + b);
      }
    }
  }
}

template <int GROUP, int ACT>
static hipError_t dispatch_mt(const QmvParams& p, const QmvLaunch& l, hipStream_t s) {
  if (l.mt == 1) {
    qmv_kernel<LOWBIT_BITS, GROUP, ACT, 1><<<l.grid, l.block, 0, s>>>(p);
  } else {
    qmv_kernel<LOWBIT_BITS, GROUP, ACT, 4><<<l.grid, l.block, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <int GROUP>
static hipError_t dispatch_act(const QmvParams& p, const QmvLaunch& l, int act, hipStream_t s) {
  switch (act) {
    case ACT_F32: return dispatch_mt<GROUP, ACT_F32>(p, l, s);
    case ACT_F16: return dispatch_mt<GROUP, ACT_F16>(p, l, s);
    case ACT_BF16: return dispatch_mt<GROUP, ACT_BF16>(p, l, s);
    default: return hipErrorInvalidValue;
  }
}

#define LOWBIT_CAT2(a, b) a##b
#define LOWBIT_CAT(a, b) LOWBIT_CAT2(a, b)
hipError_t LOWBIT_CAT(launch_qmv_b, LOWBIT_BITS)(const QmvParams& p, const QmvLaunch& l,
                                                 int group, int act, hipStream_t s) {
  switch (group) {
    case 32: return dispatch_act<32>(p, l, act, s);
    case 64: return dispatch_act<64>(p, l, act, s);
    case 128: return dispatch_act<128>(p, l, act, s);
    case 256: return dispatch_act<256>(p, l, act, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lowbit
