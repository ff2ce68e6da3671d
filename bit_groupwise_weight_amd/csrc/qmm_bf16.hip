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
//
// Pipeline: three LDS stages, each holding one K step's activation tile,
// the code runs of every (wave, column tile) and the scales / zeros of every
// (wave, pass).  All of it arrives by direct global -> LDS loads issued two
// steps ahead; at the end of a step each wave waits for its own loads of the
// next step only (an exact count, since every load of the loop is issued by
// hand) and then meets the others at a barrier without a fence.  Per-lane
// load offsets are fixed for the whole loop: each step adds one scalar base.
// The A fragments of the next (chunk, k-sub) slot are read from LDS before
// the MFMAs of the current one.
#include "qmm_common.h"

// the direct loads below name M0, which the compiler reserves, as clobbered
#pragma clang diagnostic ignored "-Winline-asm"

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

// ---- direct global -> LDS loads, issued and counted by hand
//
// Every global load of the main loop is a direct load into LDS written in
// inline assembly: the kernel then knows exactly how many of its loads are
// in flight, and before each barrier waits (vmcnt) only for the loads of the
// next step, never for those of the step after it.  (A compiler-placed wait
// cannot be that precise here: a fence drains every load, and the compiler
// does not track which stage a direct load writes across the loop.)  Lane l
// of a 16-byte load writes LDS at M0 + 16 l; of a 4- or 2-byte load, at
// M0 + 4 l (2 bytes zero-extended).

// global_load_lds_dwordx4 with a scalar base and a 32-bit lane offset
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
               : : "v"(voff), "s"(m0), "s"(sbase) : "memory", "m0");
}
// global_load_lds_dwordx4 with a 64-bit lane address
__device__ __forceinline__ void dma16_v(const void* vaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               : : "v"(vaddr), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, %2"
               : : "v"(voff), "s"(m0), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4_v(const void* vaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               : : "v"(vaddr), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma2_v(const void* vaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
               : : "v"(vaddr), "s"(m0) : "memory", "m0");
}
// Wait until at most N of this wave's loads are in flight and its LDS
// accesses are done, then meet the other waves.  No fence: the memory
// clobber alone keeps the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void wait_loads_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Code words of a run as direct loads: a 16-byte piece for the first four
// words when there are four or more, single words for the rest.
template <int BITS> struct CodePieces {
  static constexpr int x4 = BITS >= 4 ? 1 : 0;          // one 16-byte piece (words 0..3)
  static constexpr int singles = BITS - 4 * x4;         // then one word each
  static constexpr int count = x4 + singles;            // loads per run
};

template <int BITS, int MTT, int NT, int NP>
__global__ __launch_bounds__(256, 1) void qmm_bf16_kernel(QmmParams p) {
  static_assert(NT == 2, "the scale / zero loads pack 2 column tiles x 16 columns x (s, z) into 64 lanes");
  constexpr int WC = 4;
  constexpr int MC = MTT < 4 ? MTT : 4;       // row tiles per chunk
  constexpr int LPP = 4 / NP;                 // lane groups per pass
  // one pipeline stage: the activation tile, then the code runs of each
  // (wave, column tile), then the scales / zeros of each (wave, pass)
  constexpr int XBYTES = MTT * 16 * 16 * 16;
  constexpr int CBYTES = WC * NT * 256 * BITS;
  constexpr int SBYTES = WC * NP * 256;
  constexpr int STAGE = XBYTES + CBYTES + SBYTES;
  constexpr int NSTAGE = 3;
  constexpr int XSUM = 2 * NP * MTT * 4 * 16;  // [step parity][pass][row quad] float4
  constexpr int LOADS = MTT + NT * CodePieces<BITS>::count + NP;   // direct loads per step and wave
  static_assert(NSTAGE * STAGE + XSUM <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint4 smem[(NSTAGE * STAGE + XSUM) / 16];

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
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem)));
  float4_t* xsum = reinterpret_cast<float4_t*>(reinterpret_cast<char*>(smem) + NSTAGE * STAGE);

  // ---- per-lane load offsets (fixed for the whole K loop)
  // activations: load i of this wave fills rows 4q .. 4q+3 (q = WC i + wave)
  // of the tile, lane l row 4q + l/16, LDS chunk l%16 <- global chunk
  // (l%16) ^ swizzle(row)
  uint32_t xoff[MTT];                         // bytes from the step's first column
  int xrowc[MTT], xch[MTT];
#pragma unroll
  for (int i = 0; i < MTT; ++i) {
    const int row = 4 * (WC * i + wave) + (lane >> 4);
    xch[i] = 8 * ((lane & 15) ^ stage_swizzle(row & 15));
    xrowc[i] = min(m0 + row, p.M - 1);
    xoff[i] = static_cast<uint32_t>(2 * (static_cast<int64_t>(xrowc[i]) * p.K + xch[i]));
  }
  // codes: this lane's run (lane group g) of column n of each column tile
  uint32_t coff[NT];
  int ncl[NT];
  uint32_t nok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * NT * wave + 16 * nt + fr;
    nok[nt] = 0u - static_cast<uint32_t>(n < p.N);
    ncl[nt] = min(n, p.N - 1);
    coff[nt] = static_cast<uint32_t>(static_cast<int64_t>(ncl[nt]) * p.row_bytes + 4 * g * BITS);
  }
  // scales / zeros: lane L loads (L < 32 ? scale : zero) of column
  // 16 (L/16 % 2) + L%16 of this wave's columns
  const uint16_t* szp;
  {
    const int n = min(n0 + 16 * NT * wave + 16 * ((lane >> 4) & 1) + fr, p.N - 1);
    szp = static_cast<const uint16_t*>(lane < 32 ? p.scales : p.zeros) + static_cast<int64_t>(n) * p.groups;
  }

  // ---- issue the direct loads of step u into stage st (LOADS per wave)
  auto issue = [&](int u, int st) {
    const int step = s_begin + u;
    const int kb = step * QMM_BK;
    const uint32_t sb = lds0 + st * STAGE;
    const bool tail = kb + QMM_BK > p.K;      // block-uniform: only a ragged last step
    if (!tail) {
      const char* xb = static_cast<const char*>(p.x) + 2 * static_cast<int64_t>(kb);
#pragma unroll
      for (int i = 0; i < MTT; ++i) dma16_s(xoff[i], xb, sb + (WC * i + wave) * 1024);
      const uint8_t* cb = p.packed + static_cast<int64_t>(step) * 16 * BITS;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t cl = sb + XBYTES + (wave * NT + nt) * 256 * BITS;
        if constexpr (CodePieces<BITS>::x4) dma16_s(coff[nt], cb, cl);
#pragma unroll
        for (int j = 0; j < CodePieces<BITS>::singles; ++j) {
          const int wo = 4 * CodePieces<BITS>::x4 + j;
          dma4_s(coff[nt], cb + 4 * wo, cl + 256 * wo);
        }
      }
    } else {
      // ragged last step: clamp every address into its row
#pragma unroll
      for (int i = 0; i < MTT; ++i)
        dma16_v(static_cast<const char*>(p.x) +
                    2 * (static_cast<int64_t>(xrowc[i]) * p.K + min(kb + xch[i], p.K - 8)),
                sb + (WC * i + wave) * 1024);
      const int kc = min(kb + 32 * g, p.K - 32);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t cl = sb + XBYTES + (wave * NT + nt) * 256 * BITS;
        const uint8_t* src = p.packed + static_cast<int64_t>(ncl[nt]) * p.row_bytes + (kc >> 3) * BITS;
        if constexpr (CodePieces<BITS>::x4) dma16_v(src, cl);
#pragma unroll
        for (int j = 0; j < CodePieces<BITS>::singles; ++j) {
          const int wo = 4 * CodePieces<BITS>::x4 + j;
          dma4_v(src + 4 * wo, cl + 256 * wo);
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int kp = min(kb + pp * gstep, p.K - 1);
      dma2_v(szp + (kp >> p.group_shift), sb + XBYTES + CBYTES + (wave * NP + pp) * 256);
    }
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
        const float4_t xv = xsum[(parity * NP + pp) * (MTT * 4) + 4 * mt + g];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) tot[mt][nt][i] = __builtin_fmaf(zs[nt], xv[i], tot[mt][nt][i]);
      }
    }
  };

  // ---- prologue: steps 0 and 1 in flight, step 0 landed everywhere
  issue(0, 0);
  if (nsteps > 1) {
    issue(1, 1);
    wait_loads_then_barrier<LOADS>();
  } else {
    wait_loads_then_barrier<0>();
  }

  int st = 0;                                  // stage of step u
  for (int u = 0; u < nsteps; ++u) {
    const bool more = u + 2 < nsteps;          // block-uniform
    if (more) issue(u + 2, st == 0 ? 2 : st - 1);
    const int par = u & 1;
    const char* sbase = reinterpret_cast<const char*>(smem) + st * STAGE;
    const uint4* cur = reinterpret_cast<const uint4*>(sbase);

    // scales and zeros of this lane's column in each column tile and pass
    float sf[NT][NP], zf[NT][NP];
    {
      const uint32_t* szl = reinterpret_cast<const uint32_t*>(sbase + XBYTES + CBYTES) + wave * NP * 64;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int kp = (s_begin + u) * QMM_BK + pp * gstep;
        const uint32_t kok = 0u - static_cast<uint32_t>(kp < p.K);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t ok = nok[nt] & kok;
          sf[nt][pp] = bf16_bits_to_float(szl[pp * 64 + 16 * nt + fr] & ok);
          zf[nt][pp] = bf16_bits_to_float(szl[pp * 64 + 32 + 16 * nt + fr] & ok);
        }
      }
    }
    // this lane's code words and the B operands of the four k-subs
    u32x4_t bq[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const char* cl = sbase + XBYTES + (wave * NT + nt) * 256 * BITS;
      uint32_t w[BITS];
      if constexpr (CodePieces<BITS>::x4) {
        const uint4 v = reinterpret_cast<const uint4*>(cl)[lane];
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      }
#pragma unroll
      for (int j = 0; j < CodePieces<BITS>::singles; ++j) {
        const int wo = 4 * CodePieces<BITS>::x4 + j;
        w[wo] = reinterpret_cast<const uint32_t*>(cl + 256 * wo)[lane];
      }
      bq[nt][0] = code_operand<BITS, 0>(w);
      bq[nt][1] = code_operand<BITS, 1>(w);
      bq[nt][2] = code_operand<BITS, 2>(w);
      bq[nt][3] = code_operand<BITS, 3>(w);
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
      // slots t = 4 c + ks over the chunks c and k-subs ks; the A fragments
      // of slot t+1 are read before the MFMAs of slot t (two buffers), so
      // the MFMAs wait on reads issued one slot earlier
      constexpr int T = (MTT / MC) * 4;
      const bool xw = MC == WC || wave < MC;    // wave-uniform: this wave computes X of a tile
      u32x4_t fa[2][MC + 1];
      auto read_slot = [&](int t, u32x4_t (&f)[MC + 1]) {
        const int c = t >> 2, ks = t & 3;
        const int chunk = (4 * g + ks) ^ stage_swizzle(fr);
#pragma unroll
        for (int j = 0; j < MC; ++j)
          f[j] = reinterpret_cast<const u32x4_t*>(cur)[(16 * (MC * c + j) + fr) * 16 + chunk];
        if (xw)
          f[MC] = reinterpret_cast<const u32x4_t*>(cur)[(16 * (MC * c + wave) + fr) * 16 + chunk];
      };
      read_slot(0, fa[0]);
      float4_t P[MC][NT];
      float4_t Xa;
      static_for<T>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int c = t / 4, ks = t % 4;
        if constexpr (t + 1 < T) read_slot(t + 1, fa[(t + 1) % 2]);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4_t(&f)[MC + 1] = fa[t % 2];
#pragma unroll
        for (int j = 0; j < MC; ++j)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            P[j][nt] = mfma_bf16(f[j], NP == 1 ? bq[nt][ks] : (bq[nt][ks] & pm),
                                 ks == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : P[j][nt]);
        if (xw) Xa = mfma_bf16(f[MC], NP == 1 ? ones : (ones & pm), ks == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : Xa);
        if constexpr (ks == 3) {
#pragma unroll
          for (int j = 0; j < MC; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                tot[MC * c + j][nt][i] = __builtin_fmaf(sp[nt], P[j][nt][i], tot[MC * c + j][nt][i]);
          // every column of the ones product holds the row sums: the lanes of
          // column 0 publish rows 4g .. 4g+3 of the tile
          if (xw && fr == 0) xsum[(par * NP + pp) * (MTT * 4) + 4 * (MC * c + wave) + g] = Xa;
        }
      });
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) zprev[nt][pp] = zf[nt][pp];
    // step u+1 (issued one step ago) has landed in every wave's part of its
    // stage, the sums of step u are published, and stage u is read
    if (more)
      wait_loads_then_barrier<LOADS>();
    else
      wait_loads_then_barrier<0>();
    st = st == NSTAGE - 1 ? 0 : st + 1;
  }
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
  // split-K partial records, laid out as the fp16 kernel's (one K group);
  // the reduce kernel adds the planes in split order
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
