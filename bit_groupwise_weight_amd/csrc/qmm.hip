// Matrix-matrix kernel (M >= 16): y = x . dequant(Wq)^T (+ bias) on MFMA.
//
// The pages ask whether the decode approach of "metal lowbit kernels:
// qmv_fast optimization" also works for a GEMM (closing review comment), and
// the H100 table of "Add support for fbgemm int4 mm kernel" shows batched
// int4 weight-only decode falling far behind -- the batched path matters.
//
// Layout on CDNA4 (v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulation):
//   * block tile: 16*MTT rows (M) x 128 columns (N); 4 waves, wave w owns
//     columns [32w, 32w+32) as two 16-wide MFMA tiles and all M rows;
//   * K advances in steps of 128.  Within a step, lane group g = lane/16 owns
//     the 32 consecutive K positions [32g, 32g+32); MFMA slot 8g+t of k-sub
//     ks (0..3) is K position 32g + 8ks + t for both operands, so each lane's
//     weights for a step are ONE 32-code run of one row: b 32-bit words, one
//     scale and one zero (a run never crosses a group);
//   * weights are dequantized straight into MFMA operand registers
//     (w = s*q + z in fp32, rounded once to the activation type) -- every
//     column belongs to exactly one wave, so no LDS round trip is needed;
//   * the activation tile (16*MTT x 128) is shared by the 4 waves through a
//     double-buffered LDS stage filled by direct global->LDS loads (XOR
//     swizzled rows, no staging registers);
//   * the next step's codes and activations are loaded, and its weights
//     dequantized, while the current step's MFMAs run;
//   * split-K: blocks along grid.z own disjoint K ranges; with S > 1 each
//     block writes an fp32 partial plane to the workspace and a second small
//     kernel adds the planes in fixed order (results do not depend on
//     scheduling), adds the bias and rounds once.
#include "device_common.h"
#include "kernels.h"

#ifndef LOWBIT_BITS
#error "compile with -DLOWBIT_BITS=<1..7>"
#endif

namespace lowbit {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
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

constexpr int QMM_BN = 128;          // columns per block
constexpr int QMM_BK = 128;          // K per step

// Dequantize codes I and I+1 of a 32-code run into one packed pair.
template <int BITS, int ACT, int I>
__device__ __forceinline__ uint32_t dequant2(const uint32_t* w, float s, float z) {
  const float a = __builtin_fmaf(s, static_cast<float>(code_at<BITS, I>(w)), z);
  const float b = __builtin_fmaf(s, static_cast<float>(code_at<BITS, I + 1>(w)), z);
  return pack2<ACT>(a, b);
}

// Dequantize the 8 codes [8ks, 8ks+8) of a 32-code run into one operand.
template <int BITS, int ACT, int KS>
__device__ __forceinline__ uint4 dequant8(const uint32_t* w, float s, float z) {
  return make_uint4(dequant2<BITS, ACT, 8 * KS + 0>(w, s, z), dequant2<BITS, ACT, 8 * KS + 2>(w, s, z),
                    dequant2<BITS, ACT, 8 * KS + 4>(w, s, z), dequant2<BITS, ACT, 8 * KS + 6>(w, s, z));
}

// Dequantize k-sub KS (codes [8KS, 8KS+8)) of a 32-code run.
template <int BITS, int ACT, int KS>
__device__ __forceinline__ uint4 dequant_ks(const uint32_t* w, float s, float z) {
  return dequant8<BITS, ACT, KS>(w, s, z);
}

template <int BITS, int ACT>
__device__ __forceinline__ void dequant_run(const uint32_t* w, float s, float z, uint4 (&b)[4]) {
  b[0] = dequant8<BITS, ACT, 0>(w, s, z);
  b[1] = dequant8<BITS, ACT, 1>(w, s, z);
  b[2] = dequant8<BITS, ACT, 2>(w, s, z);
  b[3] = dequant8<BITS, ACT, 3>(w, s, z);
}

// Two waves per SIMD (two blocks per CU): the register budget is 256 per wave.
template <int BITS, int ACT, int MTT>
__global__ __launch_bounds__(256, 2) void qmm_kernel(QmmParams p) {
  constexpr int MROWS = 16 * MTT;
  constexpr int XCH = MTT;   // 16-byte activation chunks staged per thread per step
  // two activation stages as separate arrays, so that the compiler can tell
  // the stage being read from the one being filled
  __shared__ uint4 stage0[MTT * 16 * 16];
  __shared__ uint4 stage1[MTT * 16 * 16];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int fr = lane & 15;           // row / column inside a 16-wide MFMA tile
  const int g = lane >> 4;            // lane group: K positions [32g, 32g+32)
  const int n0 = blockIdx.x * QMM_BN;
  const int m0 = blockIdx.y * MROWS;
  const int ksteps = (p.K + QMM_BK - 1) / QMM_BK;
  const int s_begin = blockIdx.z * p.ksteps_per_split;
  const int s_end = min(ksteps, s_begin + p.ksteps_per_split);

  // ---- weight rows of this lane (clamped; out-of-range columns get s=z=0)
  int ncol[2];
  bool nok[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + 32 * wave + 16 * nt + fr;
    nok[nt] = n < p.N;
    ncol[nt] = nok[nt] ? n : p.N - 1;
  }

  auto load_codes = [&](int step, uint32_t (&w)[2][BITS], uint32_t (&sb)[2], uint32_t (&zb)[2],
                        bool& kok) {
    const int k = step * QMM_BK + 32 * g;
    kok = k < p.K;
    const int kc = kok ? k : p.K - 32;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(
          p.packed + static_cast<int64_t>(ncol[nt]) * p.row_bytes + (kc >> 3) * BITS);
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[nt][i] = src[i];
      const int64_t gi = static_cast<int64_t>(ncol[nt]) * p.groups + (kc >> p.group_shift);
      sb[nt] = static_cast<const typename Act<ACT>::bits_t*>(p.scales)[gi];
      zb[nt] = static_cast<const typename Act<ACT>::bits_t*>(p.zeros)[gi];
    }
  };
  auto dequant = [&](const uint32_t (&w)[2][BITS], const uint32_t (&sb)[2],
                     const uint32_t (&zb)[2], bool kok, uint4 (&b)[2][4]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const bool ok = kok && nok[nt];
      const float s = ok ? act_bits_to_float<ACT>(sb[nt]) : 0.0f;
      const float z = ok ? act_bits_to_float<ACT>(zb[nt]) : 0.0f;
      dequant_run<BITS, ACT>(w[nt], s, z, b[nt]);
    }
  };
  // Activation stage: the 16*MTT x 128 tile of one step, rows of 256 bytes
  // (16 chunks of 8 elements) with chunk c of row r stored at position
  // c ^ (r & 15) -- the 16 lanes that read one k-sub of an MFMA tile then hit
  // 16 different 16-byte bank groups.  It is filled with direct global->LDS
  // loads (lane i of a wave lands at dst + 16 i), so it costs no registers:
  // wave w's load i covers rows 4*(4i + w) .. +3, and each lane fetches the
  // chunk that belongs at its position.  Rows past M and chunks past K read a
  // clamped in-range address: a row past M only feeds output rows that are
  // never stored, and past K the weights are dequantized with s = z = 0.
  auto load_x_lds = [&](int step, uint4* stage) {
    uint8_t* base = reinterpret_cast<uint8_t*>(stage);
#pragma unroll
    for (int i = 0; i < MTT; ++i) {
      const int r0 = 4 * (4 * i + wave);
      const int row = r0 + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      const int grow = min(m0 + row, p.M - 1);
      const int k = min(step * QMM_BK + 8 * c, p.K - 8);
      const uint16_t* src = static_cast<const uint16_t*>(p.x) + static_cast<int64_t>(grow) * p.K + k;
      __builtin_amdgcn_global_load_lds(src, base + r0 * 256, 16, 0, 0);
    }
  };

  float4_t acc[MTT][2];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};

  // activation operands of k-sub ks (16 rows per MFMA tile, 8 K each)
  auto read_a = [&](const uint8_t* abase, int ks, uint4 (&a)[MTT]) {
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
      a[mt] = *reinterpret_cast<const uint4*>(abase + (16 * mt + fr) * 256 +
                                              (((4 * g + ks) ^ fr) << 4));
  };
  auto mma = [&](const uint4 (&bc)[2][4], int ks, const uint4 (&a)[MTT]) {
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma16x16x32<ACT>(a[mt], bc[nt][ks], acc[mt][nt]);
  };

  if (s_begin < s_end) {
    // Pipeline: codes are fetched two steps ahead (register sets A and B
    // alternate), activations one step ahead (LDS stages 0 and 1 alternate).
    // The weight operands live in one register set: right after the MFMAs of
    // k-sub ks are issued, k-sub ks of the next step is dequantized into the
    // same registers, so dequantization overlaps the remaining MFMAs.  The
    // loop always runs an even number of steps: a step past the block's
    // range loads clamped, in-range addresses and multiplies by weights
    // dequantized with s = z = 0, so it adds nothing -- keeping the loop body
    // free of branches lets the accumulators stay in place.
    uint32_t wa[2][BITS], sa[2], za[2], wb[2][BITS], sbb[2], zbb[2];
    bool ka, kb;
    uint4 bop[2][4];
    auto load_step = [&](int step, uint32_t (&w)[2][BITS], uint32_t (&sb)[2], uint32_t (&zb)[2],
                         bool& kok) {
      load_codes(min(step, s_end - 1), w, sb, zb, kok);
      kok = kok && step < s_end;
    };
    auto scale_zero = [&](const uint32_t (&sb)[2], const uint32_t (&zb)[2], bool kok, float (&sv)[2],
                          float (&zv)[2]) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bool ok = kok && nok[nt];
        sv[nt] = ok ? act_bits_to_float<ACT>(sb[nt]) : 0.0f;
        zv[nt] = ok ? act_bits_to_float<ACT>(zb[nt]) : 0.0f;
      }
    };
    load_step(s_begin, wa, sa, za, ka);
    load_x_lds(s_begin, stage0);
    load_step(s_begin + 1, wb, sbb, zbb, kb);
    dequant(wa, sa, za, ka, bop);
    __builtin_amdgcn_s_waitcnt(0);    // stage 0 has landed in LDS
    __syncthreads();

    // One K step: multiply `read` x bop; fetch the codes of step+2 into the
    // register set that just became free and the activations of step+1 into
    // `fill`; dequantize step+1 (codes already in `wn`) into bop, k-sub by
    // k-sub, behind the MFMAs that last read it.
#define LOWBIT_QMM_DQ(KS, WN, SV, ZV)                                                         \
    bop[0][KS] = dequant_ks<BITS, ACT, KS>(WN[0], SV[0], ZV[0]);                              \
    bop[1][KS] = dequant_ks<BITS, ACT, KS>(WN[1], SV[1], ZV[1]);
#define LOWBIT_QMM_STEP(STEP, READ, FILL, WN, SN, ZN, KN, WF, SF, ZF, KF)                     \
    {                                                                                        \
      load_step((STEP) + 2, WF, SF, ZF, KF);                                                 \
      load_x_lds(min((STEP) + 1, s_end - 1), FILL);                                          \
      const uint8_t* abase = reinterpret_cast<const uint8_t*>(READ);                         \
      float sv[2], zv[2];                                                                    \
      scale_zero(SN, ZN, KN, sv, zv);                                                        \
      uint4 a0[MTT], a1[MTT];                                                                \
      read_a(abase, 0, a0);                                                                  \
      read_a(abase, 1, a1);                                                                  \
      mma(bop, 0, a0);                                                                       \
      LOWBIT_QMM_DQ(0, WN, sv, zv)                                                           \
      read_a(abase, 2, a0);                                                                  \
      mma(bop, 1, a1);                                                                       \
      LOWBIT_QMM_DQ(1, WN, sv, zv)                                                           \
      read_a(abase, 3, a1);                                                                  \
      mma(bop, 2, a0);                                                                       \
      LOWBIT_QMM_DQ(2, WN, sv, zv)                                                           \
      mma(bop, 3, a1);                                                                       \
      LOWBIT_QMM_DQ(3, WN, sv, zv)                                                           \
      __builtin_amdgcn_s_waitcnt(0); /* next stage landed; this one fully read */            \
      __syncthreads();                                                                       \
    }
    for (int step = s_begin; step < s_end; step += 2) {
      LOWBIT_QMM_STEP(step, stage0, stage1, wb, sbb, zbb, kb, wa, sa, za, ka)
      LOWBIT_QMM_STEP(step + 1, stage1, stage0, wa, sa, za, ka, wb, sbb, zbb, kb)
    }
#undef LOWBIT_QMM_STEP
#undef LOWBIT_QMM_DQ
  }

  // ---- epilogue.  Lane holds D[4*g + r][fr] of each 16x16 tile.
  if (gridDim.z == 1) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = n0 + 32 * wave + 16 * nt + fr;
      if (n >= p.N) continue;
      const float bias = p.bias ? load_act<ACT>(p.bias, n) : 0.0f;
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 16 * mt + 4 * g + r;
          if (m < p.M) store_act<ACT>(p.y, static_cast<int64_t>(m) * p.N + n, acc[mt][nt][r] + bias);
        }
    }
    return;
  }

  // split-K: this block's fp32 partial sums go to plane blockIdx.z of the
  // workspace; qmm_reduce adds the planes in order.
  float* part = p.partials + static_cast<int64_t>(blockIdx.z) * p.M * p.N;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + 32 * wave + 16 * nt + fr;
    if (n >= p.N) continue;
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mt + 4 * g + r;
        if (m < p.M) part[static_cast<int64_t>(m) * p.N + n] = acc[mt][nt][r];
      }
  }
}

// y = sum over the split planes (in plane order) + bias, rounded once.
// Each thread produces 4 consecutive outputs of one row.
template <int ACT>
__global__ __launch_bounds__(256) void qmm_reduce_kernel(QmmParams p, int splits) {
  const int64_t quads_per_row = (p.N + 3) / 4;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= quads_per_row * p.M) return;
  const int m = static_cast<int>(q / quads_per_row);
  const int n = static_cast<int>(q - static_cast<int64_t>(m) * quads_per_row) * 4;
  const int64_t plane = static_cast<int64_t>(p.M) * p.N;
  const int64_t idx = static_cast<int64_t>(m) * p.N + n;
  const int cnt = min(4, p.N - n);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (cnt == 4 && (p.N % 4) == 0) {
    // planes are read four at a time so that their loads are in flight together
    int z = 0;
    for (; z + 4 <= splits; z += 4) {
      float4 t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) t[u] = *reinterpret_cast<const float4*>(p.partials + (z + u) * plane + idx);
#pragma unroll
      for (int u = 0; u < 4; ++u) { v[0] += t[u].x; v[1] += t[u].y; v[2] += t[u].z; v[3] += t[u].w; }
    }
    for (; z < splits; ++z) {
      const float4 t = *reinterpret_cast<const float4*>(p.partials + z * plane + idx);
      v[0] += t.x; v[1] += t.y; v[2] += t.z; v[3] += t.w;
    }
  } else {
    for (int z = 0; z < splits; ++z)
      for (int i = 0; i < cnt; ++i) v[i] += p.partials[z * plane + idx + i];
  }
  for (int i = 0; i < cnt; ++i) {
    const float b = p.bias ? load_act<ACT>(p.bias, n + i) : 0.0f;
    store_act<ACT>(p.y, idx + i, v[i] + b);
  }
}

template <int ACT, int MTT>
static hipError_t launch_mtt(const QmmParams& p, dim3 grid, hipStream_t s) {
  qmm_kernel<LOWBIT_BITS, ACT, MTT><<<grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <int ACT>
static hipError_t launch_act(const QmmParams& p, int mtt, dim3 grid, hipStream_t s) {
  switch (mtt) {
    case 1: return launch_mtt<ACT, 1>(p, grid, s);
    case 2: return launch_mtt<ACT, 2>(p, grid, s);
    case 4: return launch_mtt<ACT, 4>(p, grid, s);
    case 8: return launch_mtt<ACT, 8>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

#define LOWBIT_CAT2(a, b) a##b
#define LOWBIT_CAT(a, b) LOWBIT_CAT2(a, b)
hipError_t LOWBIT_CAT(launch_qmm_b, LOWBIT_BITS)(const QmmParams& p, const QmmLaunch& l, int act,
                                                 hipStream_t s) {
  hipError_t e;
  switch (act) {
    case ACT_F16: e = launch_act<ACT_F16>(p, l.mtt, l.grid, s); break;
    case ACT_BF16: e = launch_act<ACT_BF16>(p, l.mtt, l.grid, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || l.grid.z == 1) return e;
  const int64_t quads = static_cast<int64_t>(p.M) * ((p.N + 3) / 4);
  const dim3 rgrid(static_cast<unsigned>((quads + 255) / 256));
  if (act == ACT_F16) qmm_reduce_kernel<ACT_F16><<<rgrid, dim3(256), 0, s>>>(p, l.grid.z);
  else qmm_reduce_kernel<ACT_BF16><<<rgrid, dim3(256), 0, s>>>(p, l.grid.z);
  return hipGetLastError();
}

}  // namespace lowbit
