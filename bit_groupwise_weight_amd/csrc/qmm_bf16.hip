// Matrix-matrix kernel for bf16 activations (M above the decode range):
// y = x . dequant(Wq)^T (+ bias) on MFMA, with the codes as MFMA operands.
// (Compiled with the MFMA results kept in ordinary VGPRs: the group sums
// are rescaled by VALU instructions, which cannot read accumulator
// registers.)
//
// The weights are NOT dequantized before the MFMA:
// rounding s*q + z to bf16 (8 significant bits) would cost up to 2^-8 of
// every |w|, and those roundings can all fall the same way.  Instead the
// codes themselves, exact in bf16, are the B operand, and each group's
// scale and zero are applied to the fp32 results:
//     y[m, n] += s[n, g] * P[m, n] + z[n, g] * X[m, g],
//     P = sum over the group of x * q (an MFMA product),
//     X = sum over the group of x     (an MFMA product with a ones operand).
// A code q < 16 in a byte is the OCP fp8 e4m3 value q * 2^-9, so one scaled
// fp8 conversion turns two byte-placed codes into two exact bf16 values;
// wider codes go through fp32.
//
// Layout: 4 column waves x NT 16-wide column tiles per wave, MTT 16-row
// tiles, K steps of 128 with the run mapping of the fp16 kernel (lane group
// g holds 32-code run g of the step for each of its columns; k-sub ks takes
// codes 8ks..8ks+7 of it, K position 32g + 8ks + t).  A step lies in one
// group when group >= 128.  Smaller groups are taken in NP = 128 / group
// passes over the step, each with the codes (and ones) of the other groups'
// lane groups masked to zero, so that P and X of a pass cover exactly one
// group.  X is computed once per block: the row tiles go in chunks of up to
// 4, wave w runs the ones-MFMA for tile w of each chunk, writes the sums to
// LDS, and every wave adds z * X one step later, after the barrier that
// publishes them.
#include "qmm_common.h"

#ifndef LOWBIT_BITS
#error "compile with -DLOWBIT_BITS=<1..7>"
#endif

namespace lowbit {

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t bytes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bytes, 512.0f, HI));
}

// Codes I and I+1 of a run as two exact bf16 values (low half: code I).
template <int BITS, int I>
__device__ __forceinline__ uint32_t code_pair_bf16(const uint32_t (&w)[BITS]) {
  if constexpr (BITS <= 4) {
    return fp8x2_to_bf16x2<false>(code_at<BITS, I>(w) | (code_at<BITS, I + 1>(w) << 8));
  } else {
    const uint32_t f0 = __float_as_uint(static_cast<float>(code_at<BITS, I>(w)));
    const uint32_t f1 = __float_as_uint(static_cast<float>(code_at<BITS, I + 1>(w)));
    return __builtin_amdgcn_perm(f1, f0, 0x07060302u);   // the bf16 halves of both
  }
}

// B operand of k-sub KS (codes 8KS .. 8KS+7 of the run, in order).
template <int BITS, int KS>
__device__ __forceinline__ u32x4_t code_operand(const uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    // even codes in the bytes of lo, odd codes in the bytes of hi; the
    // byte permutes interleave them into code order, two codes per half word
    const uint32_t lo = and_nibbles(w[KS]);
    const uint32_t hi = and_nibbles(w[KS] >> 4);
    const uint32_t p0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    const uint32_t p1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    return u32x4_t{fp8x2_to_bf16x2<false>(p0), fp8x2_to_bf16x2<true>(p0),
                   fp8x2_to_bf16x2<false>(p1), fp8x2_to_bf16x2<true>(p1)};
  } else {
    return u32x4_t{code_pair_bf16<BITS, 8 * KS + 0>(w), code_pair_bf16<BITS, 8 * KS + 2>(w),
                   code_pair_bf16<BITS, 8 * KS + 4>(w), code_pair_bf16<BITS, 8 * KS + 6>(w)};
  }
}

__device__ __forceinline__ float4_t mfma_bf16(u32x4_t a, u32x4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                 __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
}

template <int BITS, int MTT, int NT, int NP>
__global__ __launch_bounds__(256, 1) void qmm_bf16_kernel(QmmParams p) {
  constexpr int WC = 4;
  constexpr int STAGE = MTT * 16 * 16;        // uint4 per step's activation tile
  constexpr int MC = MTT < 4 ? MTT : 4;       // row tiles per chunk
  constexpr int LPP = 4 / NP;                 // lane groups per pass
  // two activation stages as two arrays: every access below names its
  // stage statically (the loop is unrolled by two), so the compiler can see
  // that reads of one stage never alias the direct loads into the other and
  // need not wait for those loads before reading
  __shared__ uint4 stage_a[STAGE];
  __shared__ uint4 stage_b[STAGE];
  __shared__ float4_t xsum[2][NP][MTT * 4];   // [step parity][pass][row quad]: X of 4 rows

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int lane = tid & 63;
  const int fr = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT * WC);
  const int m0 = blockIdx.y * (16 * MTT);
  const int ksteps = (p.K + QMM_BK - 1) / QMM_BK;
  const int s_begin = blockIdx.z * p.ksteps_per_split;
  const int s_end = min(ksteps, s_begin + p.ksteps_per_split);
  const int nsteps = s_end - s_begin;
  const int gstep = QMM_BK / NP;              // K per pass (the group size when < 128)

  int64_t wrow[NT], szrow[NT];
  uint32_t nok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * NT * wave + 16 * nt + fr;
    nok[nt] = 0u - static_cast<uint32_t>(n < p.N);
    const int nc = min(n, p.N - 1);
    wrow[nt] = static_cast<int64_t>(nc) * p.row_bytes;
    szrow[nt] = static_cast<int64_t>(nc) * p.groups;
  }
  const uint16_t* sc_bits = static_cast<const uint16_t*>(p.scales);
  const uint16_t* ze_bits = static_cast<const uint16_t*>(p.zeros);

  // codes of one step (this lane's run of each column tile) and the raw
  // scale / zero of each pass's group, masked to zero past K, past the
  // block's steps and past N
  struct Codes {
    uint32_t w[NT][BITS];
    uint32_t s[NT][NP], z[NT][NP];
  };
  auto load_codes = [&](int u, Codes& c) {
    const int step = s_begin + u;
    const int st = min(step, s_end - 1);
    const int kc = min(st * QMM_BK + 32 * g, p.K - 32);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      load_run_words<BITS>(p.packed + wrow[nt] + (kc >> 3) * BITS, c.w[nt]);
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int kp = st * QMM_BK + pp * gstep;
        const uint32_t ok = nok[nt] & (0u - static_cast<uint32_t>((step < s_end) & (kp < p.K)));
        const int64_t gi = szrow[nt] + (min(kp, p.K - 1) >> p.group_shift);
        c.s[nt][pp] = sc_bits[gi] & ok;
        c.z[nt][pp] = ze_bits[gi] & ok;
      }
    }
  };

  // activation stage (as in the fp16 kernel, one K group)
  constexpr int RQ = 4 * MTT;
  constexpr int XL = (RQ + WC - 1) / WC;
  const uint16_t* xrow[XL];
  int xchunk[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int q = min(WC * i + wave, RQ - 1);
    const int row = 4 * q + (lane >> 4);
    xchunk[i] = 8 * ((lane & 15) ^ stage_swizzle(row & 15));
    xrow[i] = static_cast<const uint16_t*>(p.x) + static_cast<int64_t>(min(m0 + row, p.M - 1)) * p.K;
  }
  // straight from global memory into the stage (16 bytes per lane, lane l
  // of load i of this wave landing at uint4 (WC*i + wave)*64 + l): no
  // registers hold the next step's activations
  auto dma_x = [&](int u, uint4* stage) {
    const int kb = min(s_begin + u, s_end - 1) * QMM_BK;
#pragma unroll
    for (int i = 0; i < XL; ++i)
      if (RQ % WC == 0 || WC * i + wave < RQ)    // wave-uniform
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(xrow[i] + min(kb + xchunk[i], p.K - 8)),
            (__attribute__((address_space(3))) void*)(stage + (WC * i + wave) * 64), 16, 0, 0);
  };

  // lanes of pass pp: lane groups [LPP*pp, LPP*(pp+1))
  auto pass_mask = [&](int pp) { return 0u - static_cast<uint32_t>(g / LPP == pp); };
  const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs

  float4_t tot[MTT][NT];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tot[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
  float zprev[NT][NP];

  // z * X of the previous step (published by the barrier at its end)
  auto add_offset = [&](int parity, const float (&zp)[NT][NP]) {
#pragma unroll 1
    for (int pp = 0; pp < NP; ++pp) {
      float zs[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        zs[nt] = zp[nt][0];
#pragma unroll
        for (int q = 1; q < NP; ++q) zs[nt] = pp == q ? zp[nt][q] : zs[nt];
      }
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt) {
        const float4_t xv = xsum[parity][pp][4 * mt + g];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) tot[mt][nt][i] = __builtin_fmaf(zs[nt], xv[i], tot[mt][nt][i]);
      }
    }
  };

  Codes cc, cn;
  dma_x(0, stage_a);
  load_codes(0, cc);
  __syncthreads();

  // one K step: reads stage `cur`, loads the next step into `nxt`
  auto step = [&](const int u, const uint4* cur, uint4* nxt, const int par) {
    // next step's loads, in flight during this step (the barrier at its
    // end waits for them: stage u+1 is then complete)
    dma_x(u + 1, nxt);
    load_codes(u + 1, cn);

    float sf[NT][NP], zf[NT][NP];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        sf[nt][pp] = bf16_bits_to_float(cc.s[nt][pp]);
        zf[nt][pp] = bf16_bits_to_float(cc.z[nt][pp]);
      }
    u32x4_t bq[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bq[nt][0] = code_operand<BITS, 0>(cc.w[nt]);
      bq[nt][1] = code_operand<BITS, 1>(cc.w[nt]);
      bq[nt][2] = code_operand<BITS, 2>(cc.w[nt]);
      bq[nt][3] = code_operand<BITS, 3>(cc.w[nt]);
    }
    if (u > 0) add_offset(par ^ 1, zprev);
    // row tiles in chunks of MC (the group sums P of one chunk at a time,
    // which keeps the accumulators of a 128-row tile in registers); wave w
    // computes X of row tile MC * c + w of chunk c
    // (the pass loop stays rolled: unrolled, its masked operands and
    // accumulators would not fit the register file)
#pragma unroll 1
    for (int pp = 0; pp < NP; ++pp) {
      const uint32_t pm = pass_mask(pp);
      float sp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        sp[nt] = sf[nt][0];
#pragma unroll
        for (int q = 1; q < NP; ++q) sp[nt] = pp == q ? sf[nt][q] : sp[nt];
      }
#pragma unroll
      for (int c = 0; c < MTT / MC; ++c) {
        float4_t P[MC][NT];
        float4_t Xa;
        const bool xw = MC == WC || wave < MC;    // wave-uniform
        const int xmt = MC * c + (xw ? wave : 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4_t af[MC];
#pragma unroll
          for (int j = 0; j < MC; ++j)
            af[j] = reinterpret_cast<const u32x4_t*>(cur)[(16 * (MC * c + j) + fr) * 16 +
                                                            ((4 * g + ks) ^ stage_swizzle(fr))];
#pragma unroll
          for (int j = 0; j < MC; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              P[j][nt] = mfma_bf16(af[j], NP == 1 ? bq[nt][ks] : (bq[nt][ks] & pm),
                                   ks == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : P[j][nt]);
          if (xw) {
            const u32x4_t xa = reinterpret_cast<const u32x4_t*>(cur)[(16 * xmt + fr) * 16 +
                                                                       ((4 * g + ks) ^ stage_swizzle(fr))];
            Xa = mfma_bf16(xa, NP == 1 ? ones : (ones & pm), ks == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : Xa);
          }
        }
#pragma unroll
        for (int j = 0; j < MC; ++j)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              tot[MC * c + j][nt][i] = __builtin_fmaf(sp[nt], P[j][nt][i], tot[MC * c + j][nt][i]);
        // every column of the ones product holds the row sums: the lanes of
        // column 0 publish rows 4g .. 4g+3 of the tile
        if (xw && fr == 0) xsum[par][pp][4 * xmt + g] = Xa;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) zprev[nt][pp] = zf[nt][pp];
    __syncthreads();   // stage u+1 and the sums of step u are published; stage u is read
    cc = cn;
  };
  int u = 0;
  for (; u + 2 <= nsteps; u += 2) {
    step(u, stage_a, stage_b, 0);
    step(u + 1, stage_b, stage_a, 1);
  }
  if (u < nsteps) step(u, stage_a, stage_b, 0);
  add_offset((nsteps - 1) & 1, zprev);

  // ---- epilogue (lane holds D[4g + r][fr] of each 16x16 tile)
  if (gridDim.z == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + 16 * NT * wave + 16 * nt + fr;
      if (n >= p.N) continue;
      const float bias = p.bias ? load_act<ACT_BF16>(p.bias, n) : 0.0f;
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 16 * mt + 4 * g + r;
          if (m < p.M) store_act<ACT_BF16>(p.y, static_cast<int64_t>(m) * p.N + n, tot[mt][nt][r] + bias);
        }
    }
    return;
  }
  // split-K partial records, laid out as the fp16 kernel's (one K group)
  const int64_t tile = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const int64_t plane_recs = static_cast<int64_t>(gridDim.x) * gridDim.y * (WC * MTT * NT * 64);
  float4_t* part = reinterpret_cast<float4_t*>(p.partials) + (tile * WC + wave) * (MTT * NT * 64) + lane;
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) part[blockIdx.z * plane_recs + (mt * NT + nt) * 64] = tot[mt][nt];
}

template <int MTT, int NP>
static hipError_t launch_np(const QmmParams& p, const QmmLaunch& l, hipStream_t s) {
  qmm_bf16_kernel<LOWBIT_BITS, MTT, 2, NP><<<l.grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <int MTT>
static hipError_t launch_mtt(const QmmParams& p, const QmmLaunch& l, hipStream_t s) {
  if (l.nt != 2 || l.waves != 4 || l.kgroups != 1) return hipErrorInvalidValue;
  switch (p.group_shift) {
    case 5: return launch_np<MTT, 4>(p, l, s);
    case 6: return launch_np<MTT, 2>(p, l, s);
    default: return launch_np<MTT, 1>(p, l, s);
  }
}

#define LOWBIT_CAT2(a, b) a##b
#define LOWBIT_CAT(a, b) LOWBIT_CAT2(a, b)
hipError_t LOWBIT_CAT(launch_qmm_bf16_b, LOWBIT_BITS)(const QmmParams& p, const QmmLaunch& l,
                                                      hipStream_t s) {
  switch (l.mtt) {
    case 1: return launch_mtt<1>(p, l, s);
    case 2: return launch_mtt<2>(p, l, s);
    case 4: return launch_mtt<4>(p, l, s);
    case 8: return launch_mtt<8>(p, l, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lowbit
