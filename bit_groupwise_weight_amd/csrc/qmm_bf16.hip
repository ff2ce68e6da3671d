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
// codes 8ks..8ks+7 of it, K position 32g + 8ks + t).  With 128-row tiles
// the rows are split between two row groups of the 4 column waves (8 waves,
// two per SIMD).  A step lies in one group when group >= 128.  Smaller
// groups are taken in NP = 128 / group passes over the step, each with the
// codes (and ones) of the other groups' lane groups masked to zero, so that
// P and X of a pass cover exactly one group.
//
// The rescale y += s * P: the row tiles go in chunks of up to four; with an
// even chunk count a chunk's P is rescaled by the VALU while the MFMAs of
// the next chunk run (two P buffers).  The zero term z * X is itself an MFMA product: X of a row
// tile is computed once per block (by one wave), split exactly into three
// bf16 truncations and written to LDS; every four windows (pass of a step)
// one MFMA per output tile adds sum over windows and pieces of X * z.
//
// Pipeline: three LDS stages, each holding one K step's activation tile,
// the code runs of every (column wave, column tile) and the scales / zeros
// of every wave.  All of it arrives by direct global -> LDS loads issued two
// steps ahead (with one pass per step, spread over the MFMA slots); at the
// end of a step each wave waits for its own loads of the next step only (an
// exact count, since every load of the loop is issued by hand) and then
// meets the others at a barrier without a fence.  Per-lane load offsets are
// fixed for the whole loop: each step adds one scalar base.  The A
// fragments of the next (chunk, k-sub) slot are read from LDS before the
// MFMAs of the current one.
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

// LDS of one block: three pipeline stages (activation tile, code runs,
// scales / zeros of every wave) and the X pieces
constexpr int qmm_bf16_lds_bytes(int bits, int mtt, int nt, int np, int wc, int wr) {
  return 3 * (mtt * 4096 + wc * nt * 256 * bits + wc * wr * ((2 * 16 * nt * np + 63) / 64) * 256) +
         2 * mtt * 16 * 32;
}

template <int BITS, int MTT, int NT, int NP, int WC, int WR>
__global__ __launch_bounds__(64 * WC * WR, 1) void qmm_bf16_kernel(QmmParams p) {
  // WR row groups of WC column waves: wave (wr, wc) computes row tiles
  // MTW wr .. MTW wr + MTW - 1 of the columns of column wave wc
  constexpr int WV = WC * WR;                 // waves per block
  constexpr int MTW = MTT / WR;               // row tiles per wave
  static_assert(MTW >= 1 && MTT % WR == 0, "row groups");
  // row tiles per chunk: the group sums P of one chunk are in flight at a
  // time, double-buffered so that a chunk's rescale runs under the MFMAs of
  // the next (with an even chunk count per pass; otherwise right away).
  // Chunks of four: a slot's 9 MFMAs cover the LDS reads of the next slot
  // (chunks of two: 3-5 % slower at M = 128, A/B on one box)
  constexpr int MC = MTW < 4 ? MTW : 4;
  constexpr int NCH = MTW / MC;               // chunks per pass
  constexpr bool DEFER = NCH % 2 == 0;
  constexpr int LPP = 4 / NP;                 // lane groups per pass
  constexpr int CW = 16 * NT;                 // columns per wave
  constexpr int XL = 4 * MTT / WV;            // activation loads per step and wave
  static_assert((4 * MTT) % WV == 0, "every wave loads the same number of activation pieces");
  constexpr int NTL = NT / WR;                // column tiles whose codes a wave loads
  static_assert(NT % WR == 0, "code loads split between the row groups");
  // scale / zero entries of a step and wave: (pass, scale or zero, column),
  // 64 per 2-byte direct load (the last load's spare lanes repeat entries)
  constexpr int SZ_ENT = 2 * CW * NP;
  constexpr int SZ_LOADS = (SZ_ENT + 63) / 64;
  // one pipeline stage: the activation tile, then the code runs of each
  // (column wave, column tile), then the scales / zeros of each wave
  constexpr int XBYTES = MTT * 16 * 16 * 16;
  constexpr int CBYTES = WC * NT * 256 * BITS;
  constexpr int SBYTES = WV * SZ_LOADS * 256;
  constexpr int STAGE = XBYTES + CBYTES + SBYTES;
  constexpr int NSTAGE = 3;
  // X pieces: [set parity][row][window of the set][piece 0..2, zero] bf16
  constexpr int XROWS = MTT * 16;
  constexpr int XPBYTES = 2 * XROWS * 32;
  constexpr int LOADS = XL + NTL * CodePieces<BITS>::count + SZ_LOADS;   // direct loads per step and wave
  static_assert(NSTAGE * STAGE + XPBYTES <= 160 * 1024, "LDS");
  static_assert(NSTAGE * STAGE + XPBYTES == qmm_bf16_lds_bytes(BITS, MTT, NT, NP, WC, WR), "LDS size");
  __shared__ __attribute__((aligned(16))) uint4 smem[(NSTAGE * STAGE + XPBYTES) / 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int wr = wave / WC, wc = wave % WC;
  const int lane = tid & 63;
  const int fr = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT * WC);
  const int nw = n0 + 16 * NT * wc;           // first column of this wave
  const int m0 = blockIdx.y * (16 * MTT);
  const int ksteps = (p.K + QMM_BK - 1) / QMM_BK;
  const int s_begin = blockIdx.z * p.ksteps_per_split;
  const int s_end = min(ksteps, s_begin + p.ksteps_per_split);
  const int nsteps = s_end - s_begin;
  const int gstep = QMM_BK / NP;              // K per pass (the group size when < 128)
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem)));
  char* xpbase = reinterpret_cast<char*>(smem) + NSTAGE * STAGE;

  // ---- per-lane load offsets (fixed for the whole K loop)
  // activations: load i of this wave fills rows 4q .. 4q+3 (q = WV i + wave)
  // of the tile, lane l row 4q + l/16, LDS chunk l%16 <- global chunk
  // (l%16) ^ swizzle(row)
  uint32_t xoff[XL];                          // bytes from the step's first column
  int xrowc[XL], xch[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int row = 4 * (WV * i + wave) + (lane >> 4);
    xch[i] = 8 * ((lane & 15) ^ stage_swizzle(row & 15));
    xrowc[i] = min(m0 + row, p.M - 1);
    xoff[i] = static_cast<uint32_t>(2 * (static_cast<int64_t>(xrowc[i]) * p.K + xch[i]));
  }
  // codes: this lane's run (lane group g) of column n of column tile
  // WR i + wr (i < NTL), loaded by this wave for the row groups of its
  // column wave
  uint32_t coff[NTL];
  int ncl[NTL];
#pragma unroll
  for (int i = 0; i < NTL; ++i) {
    const int n = nw + 16 * (WR * i + wr) + fr;
    ncl[i] = min(n, p.N - 1);
    coff[i] = static_cast<uint32_t>(static_cast<int64_t>(ncl[i]) * p.row_bytes + 4 * g * BITS);
  }
  uint32_t nok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) nok[nt] = 0u - static_cast<uint32_t>(nw + 16 * nt + fr < p.N);
  // scales / zeros: entry e = pass * 2CW + (zero ? CW : 0) + column; lane L
  // of load i takes entry (L + 64 i) % SZ_ENT, whose column and kind do not
  // depend on i (CW divides 64)
  const uint16_t* szp;
  {
    const int n = min(nw + lane % CW, p.N - 1);
    szp = static_cast<const uint16_t*>((lane / CW) % 2 ? p.zeros : p.scales) + static_cast<int64_t>(n) * p.groups;
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
      for (int i = 0; i < XL; ++i) dma16_s(xoff[i], xb, sb + (WV * i + wave) * 1024);
      const uint8_t* cb = p.packed + static_cast<int64_t>(step) * 16 * BITS;
#pragma unroll
      for (int i = 0; i < NTL; ++i) {
        const uint32_t cl = sb + XBYTES + (wc * NT + WR * i + wr) * 256 * BITS;
        if constexpr (CodePieces<BITS>::x4) dma16_s(coff[i], cb, cl);
#pragma unroll
        for (int j = 0; j < CodePieces<BITS>::singles; ++j) {
          const int wo = 4 * CodePieces<BITS>::x4 + j;
          dma4_s(coff[i], cb + 4 * wo, cl + 256 * wo);
        }
      }
    } else {
      // ragged last step: clamp every address into its row
#pragma unroll
      for (int i = 0; i < XL; ++i)
        dma16_v(static_cast<const char*>(p.x) +
                    2 * (static_cast<int64_t>(xrowc[i]) * p.K + min(kb + xch[i], p.K - 8)),
                sb + (WV * i + wave) * 1024);
      const int kc = min(kb + 32 * g, p.K - 32);
#pragma unroll
      for (int i = 0; i < NTL; ++i) {
        const uint32_t cl = sb + XBYTES + (wc * NT + WR * i + wr) * 256 * BITS;
        const uint8_t* src = p.packed + static_cast<int64_t>(ncl[i]) * p.row_bytes + (kc >> 3) * BITS;
        if constexpr (CodePieces<BITS>::x4) dma16_v(src, cl);
#pragma unroll
        for (int j = 0; j < CodePieces<BITS>::singles; ++j) {
          const int wo = 4 * CodePieces<BITS>::x4 + j;
          dma4_v(src + 4 * wo, cl + 256 * wo);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < SZ_LOADS; ++i) {
      const int pp = ((lane + 64 * i) % SZ_ENT) / (2 * CW);
      const int kp = min(kb + pp * gstep, p.K - 1);
      dma2_v(szp + (kp >> p.group_shift), sb + XBYTES + CBYTES + (wave * SZ_LOADS + i) * 256);
    }
  };

  // load I (0 <= I < LOADS) of a whole step u, in the order of issue():
  // the activation pieces, the code pieces of each column tile, then the
  // scales / zeros.  With one pass per step the loads of step u+2 are
  // spread over the MFMA slots of step u (a few per slot), so that a wave
  // never waits long for the address unit while its MFMAs could run.
  auto issue_piece = [&](int u, int st, auto ic) {
    constexpr int I = decltype(ic)::value;
    const int step = s_begin + u;
    const uint32_t sb = lds0 + st * STAGE;
    if constexpr (I < XL) {
      dma16_s(xoff[I], static_cast<const char*>(p.x) + 2 * static_cast<int64_t>(step * QMM_BK),
              sb + (WV * I + wave) * 1024);
    } else if constexpr (I < XL + NTL * CodePieces<BITS>::count) {
      constexpr int i = (I - XL) / CodePieces<BITS>::count, j = (I - XL) % CodePieces<BITS>::count;
      const uint8_t* cb = p.packed + static_cast<int64_t>(step) * 16 * BITS;
      const uint32_t cl = sb + XBYTES + (wc * NT + WR * i + wr) * 256 * BITS;
      if constexpr (CodePieces<BITS>::x4 && j == 0) {
        dma16_s(coff[i], cb, cl);
      } else {
        constexpr int wo = 4 * CodePieces<BITS>::x4 + j - CodePieces<BITS>::x4;
        dma4_s(coff[i], cb + 4 * wo, cl + 256 * wo);
      }
    } else {
      constexpr int i = I - XL - NTL * CodePieces<BITS>::count;
      const int pp = ((lane + 64 * i) % SZ_ENT) / (2 * CW);
      const int kp = min(step * QMM_BK + pp * gstep, p.K - 1);
      dma2_v(szp + (kp >> p.group_shift), sb + XBYTES + CBYTES + (wave * SZ_LOADS + i) * 256);
    }
  };

  // lanes of pass pp: lane groups [LPP*pp, LPP*(pp+1))
  auto pass_mask = [&](int pp) { return 0u - static_cast<uint32_t>(g / LPP == pp); };
  const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs

  float4_t tot[MTW][NT];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tot[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};

  // ---- the zero term z * X as an MFMA product
  // A window is one pass of one step (a group, or the part of a group in
  // the step); four consecutive windows make a set.  The wave that computes
  // X of a row tile splits each row's X exactly into three bf16 truncations
  // (X = h0 + h1 + h2) and writes them to the set's half of XP; each lane
  // keeps z of its column for the window of its lane group (zc).  Once a
  // set is complete, one MFMA per output tile adds
  //     sum over windows w and pieces h of XP[row][w][h] * z[n][w]:
  // lane group g carries window g, A entries (h0, h1, h2, 0, 0, 0, 0, 0),
  // B entries (z, z, z, 0, 0, 0, 0, 0); products of bf16 values are exact.
  uint32_t zc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) zc[nt] = 0;
  // lane (fr, g) of the X wave writes piece fr/4 (a zero for fr/4 == 3) of
  // row 4g + fr%4 of the tile
  const int xpiece = fr >> 2;
  const int xrow_in = 4 * g + (fr & 3);
  auto publish_x = [&](const float4_t& xa, int mt, int win) {
    float v = xa[0];
    v = (fr & 3) == 1 ? xa[1] : v;
    v = (fr & 3) == 2 ? xa[2] : v;
    v = (fr & 3) == 3 ? xa[3] : v;
    const uint32_t b0 = __float_as_uint(v);
    const uint32_t h0 = b0 & 0xffff0000u;
    const float r1 = v - __uint_as_float(h0);
    const uint32_t h1 = __float_as_uint(r1) & 0xffff0000u;
    const uint32_t h2 = __float_as_uint(r1 - __uint_as_float(h1));
    uint32_t h = xpiece == 0 ? h0 : xpiece == 1 ? h1 : h2;
    h = xpiece == 3 ? 0u : h;
    const int set = (win >> 2) & 1, wi = win & 3;
    reinterpret_cast<uint16_t*>(xpbase)[((set * XROWS + 16 * mt + xrow_in) * 4 + wi) * 4 + xpiece] =
        static_cast<uint16_t>(h >> 16);
  };
  auto flush_zero_term = [&](int set) {
    u32x4_t zb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) zb[nt] = u32x4_t{zc[nt] | (zc[nt] << 16), zc[nt], 0u, 0u};
    const uint2* xp = reinterpret_cast<const uint2*>(xpbase) + (set * XROWS + 16 * MTW * wr + fr) * 4 + g;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      const uint2 a = xp[mt * 16 * 4];
      const u32x4_t av = {a.x, a.y, 0u, 0u};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) tot[mt][nt] = mfma_bf16(av, zb[nt], tot[mt][nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) zc[nt] = 0;
  };
  // windows not written before the last flush of a partial set must hold
  // finite values (their z is zero)
  for (int i = tid; i < XPBYTES / 16; i += 64 * WV)
    reinterpret_cast<uint4*>(xpbase)[i] = uint4{0u, 0u, 0u, 0u};

  // group sums of the chunks in flight, and the scale of the previous pass
  float4_t P[2][MC][NT];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < MC; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) P[b][j][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
  float sprev[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) sprev[nt] = 0.f;
  // X of the MC row tiles of chunk c of a row group comes from the MC
  // column waves of role c % NROLE (role = wc / MC), tile MC c + wc % MC;
  // the pass loop is compiled once per role, so that no branch splits the
  // MFMA stream
  constexpr int NROLE = WC / MC;
  static_assert(WC % MC == 0, "roles");
  const int role = (wc / MC) % NROLE;
  const int xtile_off = wc % MC;
  const int mt0 = MTW * wr;                   // first row tile of this wave

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
    const int st2 = st == 0 ? 2 : st - 1;      // stage of step u+2
    // spread step u+2's loads over this step's slots when it is whole
    const bool spread = NP == 1 && more && (s_begin + u + 3) * QMM_BK <= p.K;
    if (more && !spread) issue(u + 2, st2);
    const char* sbase = reinterpret_cast<const char*>(smem) + st * STAGE;
    const uint4* cur = reinterpret_cast<const uint4*>(sbase);

    // a completed set of windows (the barrier at the end of the last step
    // published its X pieces)
    if (u > 0 && ((u * NP) & 3) == 0) flush_zero_term(((u * NP - 1) >> 2) & 1);

    // zeros (bf16 bits) of this lane's column in each column tile, kept for
    // the window of this lane's group; scales are read per pass below
    const uint32_t* szl = reinterpret_cast<const uint32_t*>(sbase + XBYTES + CBYTES) + wave * SZ_LOADS * 64;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int kp = (s_begin + u) * QMM_BK + pp * gstep;
      const uint32_t kok = 0u - static_cast<uint32_t>(kp < p.K);
      const bool mine = g == ((u * NP + pp) & 3);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t zb = szl[pp * 2 * CW + CW + 16 * nt + fr] & nok[nt] & kok & 0xffffu;
        zc[nt] = mine ? zb : zc[nt];
      }
    }
    // this lane's code words and the B operands of the four k-subs
    u32x4_t bq[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const char* cl = sbase + XBYTES + (wc * NT + nt) * 256 * BITS;
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
    // row tiles in chunks of MC
    // (the pass loop stays rolled: unrolled, its masked operands and
    // accumulators would not fit the register file)
    auto passes = [&](auto role_c) __attribute__((always_inline)) {
    constexpr int ROLE = decltype(role_c)::value;
    auto xw = [](int c) { return c % NROLE == ROLE; };
    auto xtile = [&](int c) { return MC * c + xtile_off; };
#pragma unroll 1
    for (int pp = 0; pp < NP; ++pp) {
      const uint32_t pm = pass_mask(pp);
      float sp[NT];
      {
        const int kp = (s_begin + u) * QMM_BK + pp * gstep;
        const uint32_t kok = 0u - static_cast<uint32_t>(kp < p.K);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sp[nt] = bf16_bits_to_float(szl[pp * 2 * CW + 16 * nt + fr] & nok[nt] & kok);
      }
      // slots t = 4 c + ks over the chunks c and k-subs ks; the A fragments
      // of slot t+1 are read before the MFMAs of slot t (two buffers), so
      // the MFMAs wait on reads issued one slot earlier
      constexpr int T = NCH * 4;
      u32x4_t fa[2][MC + 1];
      auto read_slot = [&](int t, u32x4_t (&f)[MC + 1]) {
        const int c = t >> 2, ks = t & 3;
        const int chunk = (4 * g + ks) ^ stage_swizzle(fr);
#pragma unroll
        for (int j = 0; j < MC; ++j)
          f[j] = reinterpret_cast<const u32x4_t*>(cur)[(16 * (mt0 + MC * c + j) + fr) * 16 + chunk];
        if (xw(c))
          f[MC] = reinterpret_cast<const u32x4_t*>(cur)[(16 * (mt0 + xtile(c)) + fr) * 16 + chunk];
      };
      read_slot(0, fa[0]);
      float4_t Xa;
      static_for<T>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int c = t / 4, ks = t % 4;
        constexpr int pb = c % 2;              // P buffer of this chunk
        if constexpr (t + 1 < T) read_slot(t + 1, fa[(t + 1) % 2]);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4_t(&f)[MC + 1] = fa[t % 2];
#pragma unroll
        for (int j = 0; j < MC; ++j)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            P[pb][j][nt] = mfma_bf16(f[j], NP == 1 ? bq[nt][ks] : (bq[nt][ks] & pm),
                                     ks == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : P[pb][j][nt]);
        if (xw(c)) Xa = mfma_bf16(f[MC], NP == 1 ? ones : (ones & pm), ks == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : Xa);
        if constexpr (DEFER) {
          // rescale the previous chunk (the last one of the previous pass
          // or step when c == 0), a quarter of its tiles per k-sub
          constexpr int PAIRS = MC * NT;
          constexpr int PER = (PAIRS + 3) / 4;
#pragma unroll
          for (int q = ks * PER; q < (ks + 1) * PER && q < PAIRS; ++q) {
            const int j = q / NT, nt = q % NT;
            const int mt = MC * (c == 0 ? NCH - 1 : c - 1) + j;
            const float sc = c == 0 ? sprev[nt] : sp[nt];
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[mt][nt][i] = __builtin_fmaf(sc, P[1 - pb][j][nt][i], tot[mt][nt][i]);
          }
        }
        if constexpr (ks == 3) {
          if constexpr (!DEFER) {
#pragma unroll
            for (int j = 0; j < MC; ++j)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  tot[MC * c + j][nt][i] = __builtin_fmaf(sp[nt], P[pb][j][nt][i], tot[MC * c + j][nt][i]);
          }
          // every column of the ones product holds the row sums
          if (xw(c)) publish_x(Xa, mt0 + xtile(c), u * NP + pp);
        }
        if constexpr (NP == 1) {
          constexpr int PER = (LOADS + T - 1) / T;
          if constexpr (t * PER < LOADS) {
            __builtin_amdgcn_sched_barrier(0);
            if (spread)
              static_for<PER>([&](auto k) {
                constexpr int I = t * PER + decltype(k)::value;
                if constexpr (I < LOADS) issue_piece(u + 2, st2, std::integral_constant<int, I>{});
              });
          }
        }
      });
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sprev[nt] = sp[nt];
    }
    };
    static_for<NROLE>([&](auto r) {
      if (role == decltype(r)::value) passes(r);
    });
    // step u+1 (issued one step ago) has landed in every wave's part of its
    // stage, this step's X pieces are published, and stage u is read
    if (more)
      wait_loads_then_barrier<LOADS>();
    else
      wait_loads_then_barrier<0>();
    st = st == NSTAGE - 1 ? 0 : st + 1;
  }
  if constexpr (DEFER) {
#pragma unroll
    for (int j = 0; j < MC; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          tot[MC * (NCH - 1) + j][nt][i] = __builtin_fmaf(sprev[nt], P[1][j][nt][i], tot[MC * (NCH - 1) + j][nt][i]);
  }
  if (nsteps > 0) flush_zero_term(((nsteps * NP - 1) >> 2) & 1);

  // ---- epilogue (lane holds D[4g + r][fr] of each 16x16 tile)
  if (gridDim.z == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nw + 16 * nt + fr;
      if (n >= p.N) continue;
      const float bias = p.bias ? load_act<ACT_BF16>(p.bias, n) : 0.0f;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 16 * (mt0 + mt) + 4 * g + r;
          if (m < p.M) store_act<ACT_BF16>(p.y, static_cast<int64_t>(m) * p.N + n, tot[mt][nt][r] + bias);
        }
    }
    return;
  }
  // split-K partial records, laid out as the fp16 kernel's (one K group);
  // the reduce kernel adds the planes in split order
  const int64_t tile = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const int64_t plane_recs = static_cast<int64_t>(gridDim.x) * gridDim.y * (WC * MTT * NT * 64);
  float4_t* part = reinterpret_cast<float4_t*>(p.partials) + (tile * WC + wc) * (MTT * NT * 64) + lane;
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) part[blockIdx.z * plane_recs + ((mt0 + mt) * NT + nt) * 64] = tot[mt][nt];
}

// Two row groups where they fit LDS (their scale / zero stages are per
// wave), else one; both write the same partial-record layout.
template <int MTT, int NT, int NP, int WC>
static hipError_t launch_wr(const QmmParams& p, const QmmLaunch& l, hipStream_t s) {
  if constexpr (MTT >= 4 && NT % 2 == 0 && qmm_bf16_lds_bytes(LOWBIT_BITS, MTT, NT, NP, WC, 2) <= 160 * 1024) {
    if (l.rgroups == 2) {
      qmm_bf16_kernel<LOWBIT_BITS, MTT, NT, NP, WC, 2><<<l.grid, dim3(128 * WC), 0, s>>>(p);
      return hipGetLastError();
    }
  }
  qmm_bf16_kernel<LOWBIT_BITS, MTT, NT, NP, WC, 1><<<l.grid, dim3(64 * WC), 0, s>>>(p);
  return hipGetLastError();
}

template <int MTT, int NT, int WC>
static hipError_t launch_np(const QmmParams& p, const QmmLaunch& l, hipStream_t s) {
  switch (p.group_shift) {
    case 5: return launch_wr<MTT, NT, 4, WC>(p, l, s);
    case 6: return launch_wr<MTT, NT, 2, WC>(p, l, s);
    default: return launch_wr<MTT, NT, 1, WC>(p, l, s);
  }
}

// 128 columns per block: 4 column waves of two column tiles, in one row
// group or (64- and 128-row tiles) two
template <int MTT>
static hipError_t launch_mtt(const QmmParams& p, const QmmLaunch& l, hipStream_t s) {
  if (l.kgroups != 1 || l.waves != 4 || (l.rgroups == 2 && (MTT < 4 || l.nt != 2))) return hipErrorInvalidValue;
  if (l.nt == 1) return launch_np<MTT, 1, 4>(p, l, s);
  if (l.nt != 2) return hipErrorInvalidValue;
  return launch_np<MTT, 2, 4>(p, l, s);
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
