// Matrix-matrix kernel (M above the decode range): y = x . dequant(Wq)^T (+ bias) on MFMA.
//
// The pages ask whether the decode approach of "metal lowbit kernels:
// qmv_fast optimization" also works for a GEMM (closing review comment), and
// the H100 table of "Add support for fbgemm int4 mm kernel" shows batched
// int4 weight-only decode falling far behind -- the batched path matters.
//
// Layout on CDNA4 (v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulation):
//   * block tile: 16*MTT rows (M) x 16*NT*WC columns (N); WC column waves
//     (4 or 8), column wave c owns NT (2, or 1 for narrow tiles) 16-wide
//     column tiles and all M rows; one block per CU;
//   * K advances in steps of 128.  Within a step, lane group g = lane/16 owns
//     the 32 consecutive K positions [32g, 32g+32); MFMA slot 8g+t of k-sub
//     ks (0..3) is K position 32g + 8ks + t for both operands, so each lane's
//     weights for a step are ONE 32-code run per column tile: b 32-bit
//     words, one scale and one zero (a run never crosses a group);
//   * weights are dequantized straight into MFMA operand registers
//     (w = s*q + z in fp32, rounded once to the activation type) -- every
//     column belongs to exactly one wave, so no LDS round trip is needed;
//     4-bit codes are split into even / odd byte planes so that each code
//     converts straight from a byte;
//   * the activation tile (16*MTT x 128) is shared by the waves through two
//     LDS stages (rows swizzled by XOR); it is loaded into registers two
//     steps ahead (one with two K groups) and stored into the next stage
//     while the current one is read;
//   * codes are loaded two steps ahead; the MFMAs of each k-sub are issued
//     in a fixed order with the dequantization of the next k-sub spread
//     between them;
//   * K split inside the block (KGR = 2): two groups of waves share the
//     block tile and take alternate K steps; one LDS stage then holds the
//     tiles of both steps, and at the end the second group's accumulators
//     are added to the first group's through LDS (fixed order).  Two waves
//     per SIMD at the column width of a 4-wave block: one wave's
//     dequantization runs under the other's MFMAs without the wider tile
//     that would double the K split across blocks;
//   * split-K: blocks along grid.z own disjoint K ranges; with S > 1 each
//     block writes an fp32 partial plane to the workspace and a second small
//     kernel adds the planes in fixed order (results do not depend on
//     scheduling), adds the bias and rounds once.
#include "qmm_common.h"

#ifndef LOWBIT_BITS
#error "compile with -DLOWBIT_BITS=<1..7>"
#endif

namespace lowbit {

// Scale and zero of one 32-code run: as fp32 values, and (fp16 activations)
// as packed pairs of the fp16 bits, (s, s) and (z, z).
struct ScaleZero {
  float s, z;
  uint32_t s2, z2;
};

// Dequantize codes I and I+1 of a 32-code run into one packed pair.
template <int BITS, int ACT, int I>
__device__ __forceinline__ uint32_t dequant2(const uint32_t* w, const ScaleZero& sz) {
  const float a = __builtin_fmaf(sz.s, static_cast<float>(code_at<BITS, I>(w)), sz.z);
  const float b = __builtin_fmaf(sz.s, static_cast<float>(code_at<BITS, I + 1>(w)), sz.z);
  return pack2<ACT>(a, b);
}

// fp16 activations, 4-bit codes: byte J of the even-code plane `lo` and of
// the odd-code plane `hi` become one packed pair in packed fp16 arithmetic.
// With the exponent field of 1024 OR-ed above it, a code q in the low bits
// of a half reads as the fp16 value 1024 + q; subtracting 1024 is exact, and
// one packed FMA gives s*q + z rounded once to fp16 (the fp32 path rounds
// s*q + z to fp32 first, then to fp16).
template <int J>
__device__ __forceinline__ uint32_t dq_pair_f16_b4(uint32_t lo, uint32_t hi, const ScaleZero& sz) {
  // byte 0 = lo byte J, byte 2 = hi byte J, bytes 1 and 3 = 0
  constexpr uint32_t sel = J | (0x0Cu << 8) | ((4u + J) << 16) | (0x0Cu << 24);
  const uint32_t v = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
  const half2v_t q = __builtin_bit_cast(half2v_t, v) - half2v_t{1024, 1024};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, __builtin_bit_cast(half2v_t, sz.s2),
                                                                __builtin_bit_cast(half2v_t, sz.z2)));
}

// Dequantize k-sub KS (codes [8KS, 8KS+8)) of a 32-code run into one MFMA
// operand: four packed pairs (code 8KS+2j in the low half of dword j).
// fp16 activations, any width: codes I = 8KS+2J and I+1 are 2*BITS adjacent
// bits of the run (crossing at most one word boundary); a field extract (a
// funnel shift first where they cross) and one shift-or put them in the low
// bits of the two halves, then the packed steps of dq_pair_f16_b4.
template <int BITS, int KS, int J>
__device__ __forceinline__ uint32_t dq_pair_f16_bits(const uint32_t (&w)[BITS], const ScaleZero& sz) {
  constexpr int bit = (8 * KS + 2 * J) * BITS;
  constexpr int wi = bit / 32, off = bit % 32;
  // the two codes alone (nothing above them, which the shift-or would carry
  // into the high half)
  uint32_t x;
  if constexpr (off + 2 * BITS <= 32 || off == 0) {
    x = w[wi] >> off;
  } else {
    x = (w[wi] >> off) | (w[wi + 1] << (32 - off));
  }
  x &= (1u << (2 * BITS)) - 1u;
  constexpr uint32_t mask = ((1u << BITS) - 1u) * 0x10001u;
  const uint32_t v = ((x | (x << (16 - BITS))) & mask) | 0x64006400u;
  const half2v_t q = __builtin_bit_cast(half2v_t, v) - half2v_t{1024, 1024};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, __builtin_bit_cast(half2v_t, sz.s2),
                                                                __builtin_bit_cast(half2v_t, sz.z2)));
}

// fp16 activations dequantize in packed fp16 arithmetic (every width).
template <int BITS, int ACT>
constexpr bool packed_f16_dequant() { return ACT == ACT_F16; }

template <int BITS, int ACT, int KS>
__device__ __forceinline__ uint4 dequant_ksub(const uint32_t (&w)[BITS], const ScaleZero& sz) {
  if constexpr (BITS == 4) {
    // word KS holds the 8 codes as nibbles: split them into two byte planes
    // (even codes, odd codes) so that every code converts straight from a byte
    const uint32_t lo = and_nibbles(w[KS]);
    const uint32_t hi = and_nibbles(w[KS] >> 4);
    if constexpr (ACT == ACT_F16) {
      return make_uint4(dq_pair_f16_b4<0>(lo, hi, sz), dq_pair_f16_b4<1>(lo, hi, sz),
                        dq_pair_f16_b4<2>(lo, hi, sz), dq_pair_f16_b4<3>(lo, hi, sz));
    } else {
      const float s = sz.s, z = sz.z;
      return make_uint4(pack2<ACT>(__builtin_fmaf(s, ubyte<0>(lo), z), __builtin_fmaf(s, ubyte<0>(hi), z)),
                        pack2<ACT>(__builtin_fmaf(s, ubyte<1>(lo), z), __builtin_fmaf(s, ubyte<1>(hi), z)),
                        pack2<ACT>(__builtin_fmaf(s, ubyte<2>(lo), z), __builtin_fmaf(s, ubyte<2>(hi), z)),
                        pack2<ACT>(__builtin_fmaf(s, ubyte<3>(lo), z), __builtin_fmaf(s, ubyte<3>(hi), z)));
    }
  } else if constexpr (packed_f16_dequant<BITS, ACT>()) {
    return make_uint4(dq_pair_f16_bits<BITS, KS, 0>(w, sz), dq_pair_f16_bits<BITS, KS, 1>(w, sz),
                      dq_pair_f16_bits<BITS, KS, 2>(w, sz), dq_pair_f16_bits<BITS, KS, 3>(w, sz));
  } else {
    return make_uint4(dequant2<BITS, ACT, 8 * KS + 0>(w, sz), dequant2<BITS, ACT, 8 * KS + 2>(w, sz),
                      dequant2<BITS, ACT, 8 * KS + 4>(w, sz), dequant2<BITS, ACT, 8 * KS + 6>(w, sz));
  }
}

// Pair J (codes 8KS+2J and 8KS+2J+1) of k-sub KS of a 32-code run, packed
// into one operand dword.  For 4-bit codes, lo / hi are the byte planes of
// word KS (even codes, odd codes), so every code converts straight from a byte.
template <int BITS, int ACT, int KS, int J>
__device__ __forceinline__ uint32_t dq_pair(const uint32_t (&w)[BITS], uint32_t lo, uint32_t hi,
                                            const ScaleZero& sz) {
  if constexpr (BITS == 4 && ACT == ACT_F16) {
    return dq_pair_f16_b4<J>(lo, hi, sz);
  } else if constexpr (packed_f16_dequant<BITS, ACT>()) {
    return dq_pair_f16_bits<BITS, KS, J>(w, sz);
  } else if constexpr (BITS == 4) {
    return pack2<ACT>(__builtin_fmaf(sz.s, ubyte<J>(lo), sz.z), __builtin_fmaf(sz.s, ubyte<J>(hi), sz.z));
  } else {
    return dequant2<BITS, ACT, 8 * KS + 2 * J>(w, sz);
  }
}

// One block: 16*MTT rows x 16*NT*WC columns, WC column waves times KGR K
// groups (WV = WC*KGR waves, 4 or 8).  Column wave c owns columns
// [16*NT*c, 16*NT*(c+1)) as NT 16-wide MFMA tiles and all rows; K group kg
// takes steps s_begin + KGR*u + kg (u = 0, 1, ...: the block's super-steps).
// One block per CU: with 4 waves each wave has a whole SIMD's registers; with
// 8, two waves share a SIMD, so one wave's dequantization can run while the
// other's MFMAs execute.
template <int BITS, int ACT, int MTT, int NT, int WC, int KGR>
__global__ __launch_bounds__(64 * WC * KGR, 1) void qmm_kernel(QmmParams p) {
  constexpr int WV = WC * KGR;
  constexpr int STAGE = MTT * 16 * 16;   // uint4 per step's activation tile (16*MTT rows x 256 B)
  constexpr int MH = MTT > 1 ? MTT / 2 : 1;   // activation fragments are refilled in two halves
  // two stages of KGR step tiles each
  __shared__ uint4 lds[2 * KGR * STAGE];
  uint4* const stage0 = lds;
  uint4* const stage1 = lds + KGR * STAGE;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int cw = wave % WC;           // column wave
  const int kg = wave / WC;           // K group
  const int lane = tid & 63;
  const int fr = lane & 15;           // row / column inside a 16-wide MFMA tile
  const int g = lane >> 4;            // lane group: K positions [32g, 32g+32) of a step
  const int n0 = blockIdx.x * (16 * NT * WC);
  // activation row quads (4 rows x 256 bytes = one load instruction per wave)
  // per step, and how many of a super-step's KGR*RQ each wave loads
  constexpr int RQ = 4 * MTT;
  constexpr int XL = (KGR * RQ + WV - 1) / WV;
  const int m0 = blockIdx.y * (16 * MTT);
  const int ksteps = (p.K + QMM_BK - 1) / QMM_BK;
  const int s_begin = blockIdx.z * p.ksteps_per_split;
  const int s_end = min(ksteps, s_begin + p.ksteps_per_split);
  const int supers = (s_end - s_begin + KGR - 1) / KGR;
  // this wave's K step in super-step u
  auto wstep = [&](int u) { return s_begin + KGR * u + kg; };

  // ---- this lane's weight rows (clamped; columns past N get s = z = 0)
  int64_t wrow[NT], szrow[NT];
  uint32_t nok[NT];   // all ones for a real column, 0 past N
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * NT * cw + 16 * nt + fr;
    nok[nt] = 0u - static_cast<uint32_t>(n < p.N);
    const int nc = min(n, p.N - 1);
    wrow[nt] = static_cast<int64_t>(nc) * p.row_bytes;
    szrow[nt] = static_cast<int64_t>(nc) * p.groups;
  }
  using bits_t = typename Act<ACT>::bits_t;
  const bits_t* sc_bits = static_cast<const bits_t*>(p.scales);
  const bits_t* ze_bits = static_cast<const bits_t*>(p.zeros);

  // Codes of one step for this lane: NT runs of 32 codes, their scale and
  // zero (raw bits), and a mask that is all ones when the step's K range of
  // this lane group is real.  Masks, not branches: the loop stays straight.
  struct Codes {
    uint32_t w[NT][BITS];
    uint32_t s[NT], z[NT];
    uint32_t ok;
  };
  auto load_codes = [&](int step, Codes& c) {
    const int st = min(step, s_end - 1);
    const int k = st * QMM_BK + 32 * g;
    c.ok = 0u - static_cast<uint32_t>((step < s_end) & (k < p.K));
    const int kc = min(k, p.K - 32);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      load_run_words<BITS>(p.packed + wrow[nt] + (kc >> 3) * BITS, c.w[nt]);
      const int64_t gi = szrow[nt] + (kc >> p.group_shift);
      c.s[nt] = sc_bits[gi];
      c.z[nt] = ze_bits[gi];
    }
  };
  auto scale_zero = [&](const Codes& c, ScaleZero (&sz)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t ok = c.ok & nok[nt];
      const uint32_t sb = c.s[nt] & ok, zb = c.z[nt] & ok;   // zero bits -> +0.0
      if constexpr (packed_f16_dequant<BITS, ACT>()) {
        sz[nt].s2 = (sb & 0xFFFFu) * 0x10001u;
        sz[nt].z2 = (zb & 0xFFFFu) * 0x10001u;
      } else {
        sz[nt].s = act_bits_to_float<ACT>(sb);
        sz[nt].z = act_bits_to_float<ACT>(zb);
      }
    }
  };

  // Activation stage: the 16*MTT x 128 tiles of a super-step's KGR steps
  // (tile j at uint4 offset j*STAGE), rows of 256 bytes (16 chunks of 8
  // elements) with chunk c of row r stored at position c ^ stage_swizzle(r & 15)
  // (see there).  Load i of wave w covers quad q = WV*i + w of the stage: step
  // j = q / RQ of the super-step, row quad q % RQ (rows 4(q%RQ) .. +3; quads
  // past the stage are skipped): lane l fetches the chunk that belongs at
  // position l & 15 of row 4(q%RQ) + l/16, and later stores it at byte 16 l
  // of quad q.  Rows past M and chunks past K read a clamped in-range
  // address: such a row only feeds output rows that are never stored, and
  // past K (or past the block's last step) the weights are dequantized with
  // s = z = 0.
  const uint16_t* xrow[XL];
  int xchunk[XL], xstep[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int q = min(WV * i + wave, KGR * RQ - 1);
    const int row = 4 * (q % RQ) + (lane >> 4);
    xstep[i] = q / RQ;
    xchunk[i] = 8 * ((lane & 15) ^ stage_swizzle(row & 15));
    xrow[i] = static_cast<const uint16_t*>(p.x) + static_cast<int64_t>(min(m0 + row, p.M - 1)) * p.K;
  }
  // (native vectors: HIP's uint4 is a struct whose copies become memcpys
  // that keep these arrays out of registers)
  auto load_x = [&](int u, u32x4_t (&xr)[XL]) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int kb = min(s_begin + KGR * u + xstep[i], s_end - 1) * QMM_BK;
      xr[i] = *reinterpret_cast<const u32x4_t*>(xrow[i] + min(kb + xchunk[i], p.K - 8));
    }
  };
  auto store_x = [&](const u32x4_t (&xr)[XL], uint4* stage) {
#pragma unroll
    for (int i = 0; i < XL; ++i)
      if ((KGR * RQ) % WV == 0 || WV * i + wave < KGR * RQ)    // wave-uniform
        reinterpret_cast<u32x4_t*>(stage)[(WV * i + wave) * 64 + lane] = xr[i];
  };

  float4_t acc[MTT][NT];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t bw[NT][4][4];   // weight operands of the current step: [column tile][k-sub][dword]
  uint4 af[MTT];           // activation operands of one k-sub: [row tile]

  // activation operands of row tiles [MT0, MT1) for k-sub KS
  // (from this K group's tile of the stage)
  auto read_a = [&](const uint4* stage, auto KSc, auto MT0c, auto MT1c) {
    constexpr int KS = decltype(KSc)::value;
    const uint4* t = stage + (KGR > 1 ? kg * STAGE : 0);
    static_for<decltype(MT1c)::value - decltype(MT0c)::value>([&](auto ic) {
      constexpr int mt = decltype(MT0c)::value + decltype(ic)::value;
      af[mt] = t[(16 * mt + fr) * 16 + ((4 * g + KS) ^ stage_swizzle(fr))];
    });
  };
  using I0 = std::integral_constant<int, 0>;
  using IMH = std::integral_constant<int, MH>;
  using IMTT = std::integral_constant<int, MTT>;

  // One phase: the MFMAs of k-sub KS in row-tile-major order, with the
  // dequantization of k-sub DKS of code set C spread evenly between them (one
  // packed pair at a time), and the activation operands of k-sub NKS (from
  // stage NS, if NKS >= 0) read in two halves as soon as the MFMAs that use
  // their registers have been issued.  Scheduling barriers pin this order:
  // with one wave per SIMD, the MFMA pipe stays busy only if the VALU work
  // sits between the MFMAs rather than in clusters.
  auto phase = [&](auto KSc, auto DKSc, const Codes& C, const ScaleZero (&sz)[NT], const uint4* ns,
                   auto NKSc) {
    constexpr int KS = decltype(KSc)::value;
    constexpr int DKS = decltype(DKSc)::value;
    constexpr int NKS = decltype(NKSc)::value;
    constexpr int NMF = MTT * NT;
    constexpr int NPC = NT * 4;
    uint32_t lo[NT], hi[NT];
    static_for<NMF>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int mt = i / NT, nt = i % NT;
      acc[mt][nt] = mfma16x16x32<ACT>(af[mt], make_uint4(bw[nt][KS][0], bw[nt][KS][1], bw[nt][KS][2],
                                                         bw[nt][KS][3]), acc[mt][nt]);
      constexpr int p0 = i * NPC / NMF, p1 = (i + 1) * NPC / NMF;
      static_for<p1 - p0>([&](auto jc) {
        constexpr int pc = p0 + decltype(jc)::value;
        constexpr int c = pc / 4, j = pc % 4;
        if constexpr (BITS == 4 && j == 0) {
          lo[c] = and_nibbles(C.w[c][DKS]);
          hi[c] = and_nibbles(C.w[c][DKS] >> 4);
        }
        bw[c][DKS][j] = dq_pair<BITS, ACT, DKS, j>(C.w[c], lo[c], hi[c], sz[c]);
      });
      if constexpr (NKS >= 0 && i == MH * NT - 1)
        read_a(ns, std::integral_constant<int, NKS>{}, I0{}, IMH{});
      if constexpr (NKS >= 0 && MH < MTT && i == NMF - 1)
        read_a(ns, std::integral_constant<int, NKS>{}, IMH{}, IMTT{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  using K3 = std::integral_constant<int, 3>;

  // Pipeline over super-steps (one K step per wave each), with two register
  // sets (A, B) for codes and activations: super-step u reads LDS stage u%2;
  // in its first phase it loads the activations of super-step u+2 and, once
  // k-sub 3 of its own codes is dequantized, this wave's codes of super-step
  // u+2; it stores the activations of super-step u+1 into the other stage
  // and meets the other waves once that stage is written and its own is fully
  // read, then reads the first operands of super-step u+1 during its last
  // phase.  Weight operands are dequantized one k-sub ahead, in place: k-sub
  // 3 of step u during phase 0, k-subs 0..2 of step u+1 during phases 1..3.
  // With two K groups a super-step's activations take twice the registers,
  // so they use one register set: loaded one super-step ahead and stored
  // just before the barrier.  All loads are ordinary loads that complete in
  // order, so every use waits only for the loads it needs.
  constexpr bool X1 = KGR > 1;
#define LOWBIT_QMM_STEP(S_, SR, SW, XLD, XST, CUR, NXT)                                       \
  {                                                                                           \
    load_x((S_) + (X1 ? 1 : 2), XLD);                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    {                                                                                         \
      ScaleZero sz[NT];                                                                       \
      scale_zero(CUR, sz);                                                                    \
      phase(K0{}, K3{}, CUR, sz, SR, K1{});                                                   \
    }                                                                                         \
    load_codes(wstep((S_) + 2), CUR);                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    ScaleZero sz[NT];                                                                         \
    scale_zero(NXT, sz);                                                                      \
    phase(K1{}, K0{}, NXT, sz, SR, K2{});                                                     \
    if constexpr (!X1) store_x(XST, SW);                                                      \
    phase(K2{}, K1{}, NXT, sz, SR, K3{});                                                     \
    if constexpr (X1) store_x(XLD, SW);                                                       \
    __syncthreads(); /* stage S_+1 written by every wave; stage S_ fully read */              \
    phase(K3{}, K2{}, NXT, sz, SW, K0{});                                                     \
  }

  Codes ca, cb;
  u32x4_t xa[XL], xb[XL];
  load_x(0, xa);
  if constexpr (!X1) load_x(1, xb);
  load_codes(wstep(0), ca);
  load_codes(wstep(1), cb);
  store_x(xa, stage0);
  {
    ScaleZero sz[NT];
    scale_zero(ca, sz);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4 b0 = dequant_ksub<BITS, ACT, 0>(ca.w[nt], sz[nt]);
      const uint4 b1 = dequant_ksub<BITS, ACT, 1>(ca.w[nt], sz[nt]);
      const uint4 b2 = dequant_ksub<BITS, ACT, 2>(ca.w[nt], sz[nt]);
      bw[nt][0][0] = b0.x; bw[nt][0][1] = b0.y; bw[nt][0][2] = b0.z; bw[nt][0][3] = b0.w;
      bw[nt][1][0] = b1.x; bw[nt][1][1] = b1.y; bw[nt][1][2] = b1.z; bw[nt][1][3] = b1.w;
      bw[nt][2][0] = b2.x; bw[nt][2][1] = b2.y; bw[nt][2][2] = b2.z; bw[nt][2][3] = b2.w;
    }
  }
  __syncthreads();
  read_a(stage0, K0{}, I0{}, IMTT{});
  int u = 0;
  if constexpr (X1) {
    for (; u + 2 <= supers; u += 2) {
      LOWBIT_QMM_STEP(u, stage0, stage1, xa, xa, ca, cb)
      LOWBIT_QMM_STEP(u + 1, stage1, stage0, xa, xa, cb, ca)
    }
    if (u < supers) LOWBIT_QMM_STEP(u, stage0, stage1, xa, xa, ca, cb)
  } else {
    for (; u + 2 <= supers; u += 2) {
      LOWBIT_QMM_STEP(u, stage0, stage1, xa, xb, ca, cb)
      LOWBIT_QMM_STEP(u + 1, stage1, stage0, xb, xa, cb, ca)
    }
    if (u < supers) LOWBIT_QMM_STEP(u, stage0, stage1, xa, xb, ca, cb)
  }
#undef LOWBIT_QMM_STEP

  if constexpr (KGR > 1) {
    // K groups 1.. hand their sums to group 0 through LDS (the stages are no
    // longer read once every wave is past this barrier); group 0 adds them in
    // group order.  A lane's record (cw, mt, nt) sits at
    // ((cw * MTT + mt) * NT + nt) * 64 + lane of its group's region.
    static_assert((KGR - 1) * WC * MTT * NT * 64 <= 2 * KGR * STAGE, "K-group sums exceed LDS");
    float4_t* red = reinterpret_cast<float4_t*>(lds);
    __syncthreads();
    if (kg > 0) {
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          red[((((kg - 1) * WC + cw) * MTT + mt) * NT + nt) * 64 + lane] = acc[mt][nt];
    }
    __syncthreads();
#pragma unroll
    for (int j = 1; j < KGR; ++j)
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] += red[((((j - 1) * WC + cw) * MTT + mt) * NT + nt) * 64 + lane];
  }

  // ---- epilogue.  Lane holds D[4*g + r][fr] of each 16x16 tile; with K
  // groups only group 0 holds the block's sums (the other groups stay for
  // the barriers below and store nothing).
  const bool holder = (KGR == 1) || kg == 0;
  auto store_y = [&](const float4_t (&v)[MTT][NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + 16 * NT * cw + 16 * nt + fr;
      if (n >= p.N) continue;
      const float bias = p.bias ? load_act<ACT>(p.bias, n) : 0.0f;
#pragma unroll
      for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 16 * mt + 4 * g + r;
          if (m < p.M) store_act<ACT>(p.y, static_cast<int64_t>(m) * p.N + n, v[mt][nt][r] + bias);
        }
    }
  };
  if (gridDim.z == 1) {
    if (holder) store_y(acc);
    return;
  }

  // split-K: this block's fp32 partial sums go to plane blockIdx.z of the
  // workspace in tile order.  A lane's four accumulators of one 16x16 tile
  // form a 16-byte record; record (tile, wave, mt, nt, lane) sits at
  // ((((tile * WC + wave) * MTT + mt) * NT + nt) * 64 + lane), so each store
  // instruction writes 1 KB contiguous per wave and the planes need no
  // row/column arithmetic (wave = the column wave).  qmm_reduce_kernel adds
  // the planes in order.
  const int64_t tile = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const int64_t plane_recs = static_cast<int64_t>(gridDim.x) * gridDim.y * (WC * MTT * NT * 64);
  float4_t* part = reinterpret_cast<float4_t*>(p.partials) + (tile * WC + cw) * (MTT * NT * 64) + lane;
  if (holder) {
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) part[blockIdx.z * plane_recs + (mt * NT + nt) * 64] = acc[mt][nt];
  }
}

// y = sum over the split planes (in plane order) + bias, rounded once.  One
// thread per 16-byte record of the tile-order planes: D[4g + r][fr] of one
// 16x16 tile for r = 0..3 (fr = lane & 15, g = lane >> 4).
template <int ACT>
__global__ __launch_bounds__(256) void qmm_reduce_kernel(QmmParams p, QmmReduceShape r) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= r.plane_recs) return;
  const int lane = static_cast<int>(q & 63);
  const int64_t rec = q >> 6;
  const int nt = static_cast<int>(rec & ((1 << r.nt_shift) - 1));
  const int mt = static_cast<int>((rec >> r.nt_shift) & ((1 << r.mtt_shift) - 1));
  const int w = static_cast<int>((rec >> (r.nt_shift + r.mtt_shift)) & ((1 << r.wv_shift) - 1));
  const int64_t tile = rec >> (r.nt_shift + r.mtt_shift + r.wv_shift);
  const int bx = static_cast<int>(tile % r.tiles_n);
  const int by = static_cast<int>(tile / r.tiles_n);
  const int n = (bx << (4 + r.nt_shift + r.wv_shift)) + (w << (4 + r.nt_shift)) + (nt << 4) + (lane & 15);
  const int m = (by << (4 + r.mtt_shift)) + (mt << 4) + 4 * (lane >> 4);
  if (n >= p.N || m >= p.M) return;
  const float4_t* src = reinterpret_cast<const float4_t*>(p.partials) + q;
  // planes are read four at a time so that their loads are in flight together
  float4_t v = {0.f, 0.f, 0.f, 0.f};
  int z = 0;
  for (; z + 4 <= r.splits; z += 4) {
    float4_t t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = src[(z + u) * r.plane_recs];
#pragma unroll
    for (int u = 0; u < 4; ++u) v += t[u];
  }
  for (; z < r.splits; ++z) v += src[z * r.plane_recs];
  const float b = p.bias ? load_act<ACT>(p.bias, n) : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (m + i < p.M) store_act<ACT>(p.y, static_cast<int64_t>(m + i) * p.N + n, v[i] + b);
}

// Instances: 4 column waves (one K group) for every bit width; 8 waves (256
// registers per wave) -- 8 column waves up to qmm_max_bits_8waves, 4 column
// waves in two K groups up to qmm_max_bits_kgroups -- above which the code
// registers of the pipeline no longer fit without spilling.
template <int ACT, int MTT>
static hipError_t launch_mtt(const QmmParams& p, const QmmLaunch& l, hipStream_t s) {
  if (l.nt == 1) {
    if constexpr (LOWBIT_BITS <= qmm_max_bits_kgroups && MTT == 8) {
      if (l.waves == 4 && l.kgroups == 2) {
        qmm_kernel<LOWBIT_BITS, ACT, MTT, 1, 4, 2><<<l.grid, dim3(512), 0, s>>>(p);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  }
  if (l.nt != 2) return hipErrorInvalidValue;
  if (l.waves == 4 && l.kgroups == 1) {
    qmm_kernel<LOWBIT_BITS, ACT, MTT, 2, 4, 1><<<l.grid, dim3(256), 0, s>>>(p);
  } else if (l.waves == 8 && l.kgroups == 1) {
    if constexpr (LOWBIT_BITS <= qmm_max_bits_8waves) {
      qmm_kernel<LOWBIT_BITS, ACT, MTT, 2, 8, 1><<<l.grid, dim3(512), 0, s>>>(p);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (l.waves == 4 && l.kgroups == 2) {
    if constexpr (LOWBIT_BITS <= qmm_max_bits_kgroups) {
      qmm_kernel<LOWBIT_BITS, ACT, MTT, 2, 4, 2><<<l.grid, dim3(512), 0, s>>>(p);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int ACT>
static hipError_t launch_act(const QmmParams& p, const QmmLaunch& l, hipStream_t s) {
  switch (l.mtt) {
    case 1: return launch_mtt<ACT, 1>(p, l, s);
    case 2: return launch_mtt<ACT, 2>(p, l, s);
    case 4: return launch_mtt<ACT, 4>(p, l, s);
    case 8: return launch_mtt<ACT, 8>(p, l, s);
    default: return hipErrorInvalidValue;
  }
}

// ---- small M (at most 16 rows), fp16 activations
//
// At a few rows the MFMA work is small and the time goes to streaming the
// packed weights -- and, on this hardware, to the number of vector-memory
// instructions each CU must issue (a wave stalls while the address unit
// works through its queue).  So the block shape follows the decode kernel
// and every load is as wide as it can be: a block owns 16*NT columns over
// ALL of K (no K split across blocks, no second kernel), its WV waves take
// contiguous ranges of K steps, two steps per chunk, one chunk in flight
// ahead of the MFMAs.  Per step a wave loads
//   * the activation rows, 4 rows x 256 contiguous bytes per instruction
//     (MR instructions: rows past M repeat row M-1), which it writes to its
//     own LDS slice (swizzled as the tiled kernels' stage) and reads back as
//     A fragments -- one wave writes and reads, so no barrier;
//   * per column tile, this lane's 32-code run (the run mapping above);
// and per chunk the scales and zeros its runs need, spread over the four
// lanes of each column (one 2-byte load per lane per chunk at group >= 128)
// and handed to the lanes that use them by ds_bpermute.
// The waves' 16 x 16*NT partial tiles are added through LDS in wave order
// (fixed), the bias is added and the result rounded once.
template <int BITS, int NT, int WV, int MR>
__global__ __launch_bounds__(64 * WV) void qmm_small_kernel(QmmParams p) {
  constexpr int CH = 2;                        // K steps per load chunk
  __shared__ float4_t red[WV][NT][64];
  __shared__ uint4 xs[WV][4 * MR * 16];        // per wave: 4*MR rows x 16 chunks of 16 bytes
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int fr = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * (16 * NT);
  const int ksteps = (p.K + QMM_BK - 1) / QMM_BK;
  const int spw = (ksteps + WV - 1) / WV;      // steps per wave
  const int s0 = min(ksteps, wave * spw);
  const int s1 = min(ksteps, s0 + spw);
  const int gsh = p.group_shift;
  // groups per step a lane's runs fall in: R = 128 / min(group, 128)
  const int rsh = gsh >= 7 ? 0 : 7 - gsh;      // log2 R
  const int R = 1 << rsh;
  // activation pieces: piece i of a step is row min(4i + l/16, M-1), 16
  // bytes at K offset 8 (l%16); it lands at chunk (l%16) ^ swizzle(row)
  const _Float16* xp[MR];
  int xdst[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int r = 4 * i + g;
    xp[i] = static_cast<const _Float16*>(p.x) + static_cast<int64_t>(min(r, p.M - 1)) * p.K + 8 * fr;
    xdst[i] = r * 16 + (fr ^ stage_swizzle(r));
  }
  const int arow = min(fr, 4 * MR - 1);        // A fragment row (rows >= M hold row M-1)
  const uint8_t* crow[NT];
  const uint16_t* srow[NT];
  const uint16_t* zrow[NT];
  bool nok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt + fr;
    nok[nt] = n < p.N;
    const int nc = min(n, p.N - 1);
    crow[nt] = p.packed + static_cast<int64_t>(nc) * p.row_bytes;
    srow[nt] = static_cast<const uint16_t*>(p.scales) + static_cast<int64_t>(nc) * p.groups;
    zrow[nt] = static_cast<const uint16_t*>(p.zeros) + static_cast<int64_t>(nc) * p.groups;
  }

  // One chunk (steps j0, j0 + 1).  Scale / zero slots: slot q of the chunk
  // is group ((j0 + q / R) * 128 + (q % R) * min(group, 128)) >> gsh, q <
  // 2R; value v < 4R is (v < 2R ? scale : zero) of slot v % 2R, held by
  // lane group v % 4 of the column in register v / 4.
  // (loaded values are kept raw: a select on a loaded value would make the
  // load wait at once; the masks are applied where the values are used)
  struct Chunk {
    uint4 x[CH][MR];
    uint32_t xok[CH];                          // activation pieces inside K: all ones, else 0
    uint32_t w[CH][NT][BITS];
    uint32_t sz[NT][4];                        // this lane's values, by register (R of them)
    uint32_t szok[NT][4];
  };
  auto load = [&](int j0, Chunk& C) {
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int j = j0 + t;
      const int kb = j * QMM_BK;
      const bool step_ok = j < s1;
      // activation pieces (K offsets past K read zero; K is a multiple of
      // 32, so a piece is wholly inside or outside)
      const bool kin = step_ok && kb + 8 * fr < p.K;
      C.xok[t] = kin ? 0xffffffffu : 0u;
#pragma unroll
      for (int i = 0; i < MR; ++i) C.x[t][i] = *reinterpret_cast<const uint4*>(xp[i] + (kin ? kb : 0));
      const int kr = kb + 32 * g;              // this lane's run
      const int kc = (step_ok && kr < p.K) ? kr : 0;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) load_run_words<BITS>(crow[nt] + (kc >> 3) * BITS, C.w[t][nt]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        C.sz[nt][i] = 0u;
        C.szok[nt][i] = 0u;
      }
      if (i < R) {                              // wave-uniform
        const int v = 4 * i + g;
        const int q = v & (2 * R - 1);
        const int kq = (j0 + (q >> rsh)) * QMM_BK + ((q & (R - 1)) << (gsh >= 7 ? 7 : gsh));
        const bool ok = j0 + (q >> rsh) < s1 && kq < p.K;
        const int gi = ok ? (kq >> gsh) : 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          C.sz[nt][i] = (v < 2 * R ? srow[nt] : zrow[nt])[gi];
          C.szok[nt][i] = (ok && nok[nt]) ? 0xffffu : 0u;
        }
      }
    }
  };
  float4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = float4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Chunk& C) {
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      // this step's activation rows through the wave's LDS slice
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        const uint32_t m = C.xok[t];
        xs[wave][xdst[i]] = make_uint4(C.x[t][i].x & m, C.x[t][i].y & m, C.x[t][i].z & m, C.x[t][i].w & m);
      }
      uint4 a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[ks] = xs[wave][arow * 16 + ((4 * g + ks) ^ stage_swizzle(arow))];
      // scale and zero of this lane's run, slot q = t R + 32 g / min(group,
      // 128): the scale is value q, the zero value 2R + q, each held by
      // lane group (v % 4) of the column in register v / 4 -- a register
      // index that is the same for every lane (R = 4: t and 2 + t, held by
      // the lane itself; R = 2: 0 and 1; R = 1: 0 and 0)
      const int q = t * R + ((32 * g) >> (gsh >= 7 ? 7 : gsh));
      const int rs = R == 4 ? t : 0;
      const int rz = R == 4 ? 2 + t : R == 2 ? 1 : 0;
      ScaleZero sz[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        uint32_t sv = C.sz[nt][0] & C.szok[nt][0], zv = sv;
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          const uint32_t vi = C.sz[nt][i] & C.szok[nt][i];
          sv = rs == i ? vi : sv;
          zv = rz == i ? vi : zv;
        }
        if (R < 4) {                            // wave-uniform
          sv = __builtin_amdgcn_ds_bpermute(4 * (fr + 16 * (q & 3)), sv);
          zv = __builtin_amdgcn_ds_bpermute(4 * (fr + 16 * ((2 * R + q) & 3)), zv);
        }
        sz[nt].s = 0.f;
        sz[nt].z = 0.f;
        sz[nt].s2 = (sv & 0xffffu) * 0x10001u;
        sz[nt].z2 = (zv & 0xffffu) * 0x10001u;
      }
      static_for<4>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = mfma16x16x32<ACT_F16>(a[ks], dequant_ksub<BITS, ACT_F16, ks>(C.w[t][nt], sz[nt]), acc[nt]);
      });
    }
  };

  Chunk buf[2];
  if (s0 < s1) load(s0, buf[0]);
  for (int j = s0; j < s1; j += 2 * CH) {      // wave-uniform bounds
    if (j + CH < s1) load(j + CH, buf[1]);
    compute(buf[0]);
    if (j + CH >= s1) break;
    if (j + 2 * CH < s1) load(j + 2 * CH, buf[0]);
    compute(buf[1]);
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) red[wave][nt][lane] = acc[nt];
  __syncthreads();
  // wave nt (< NT) adds the column tile's WV partial tiles in wave order
  if (wave < NT) {
    float4_t v = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < WV; ++w) v += red[w][wave][lane];
    const int n = n0 + 16 * wave + fr;
    if (n < p.N) {
      const float b = p.bias ? load_act<ACT_F16>(p.bias, n) : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * g + r;
        if (m < p.M) store_act<ACT_F16>(p.y, static_cast<int64_t>(m) * p.N + n, v[r] + b);
      }
    }
  }
}

template <int NT, int MR>
static hipError_t launch_small_mr(const QmmParams& p, int waves, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.N + 16 * NT - 1) / (16 * NT)));
  // instances whose registers would spill are not built: past 4 rows or 6
  // bits no 16-wave blocks; at 7 bits, 32 columns and 16 rows 4 waves
  constexpr bool w16 = NT == 1 && MR == 1 && LOWBIT_BITS <= 6;
  constexpr bool w8 = !(NT == 2 && MR == 4 && LOWBIT_BITS > 6);
  if (waves == 16 && !w16) waves = 8;
  if (waves == 8 && !w8) waves = 4;
  switch (waves) {
    case 4: qmm_small_kernel<LOWBIT_BITS, NT, 4, MR><<<grid, dim3(256), 0, s>>>(p); break;
    case 8:
      if constexpr (w8) {
        qmm_small_kernel<LOWBIT_BITS, NT, 8, MR><<<grid, dim3(512), 0, s>>>(p);
        break;
      }
      return hipErrorInvalidValue;
    case 16:
      if constexpr (w16) {   // 1024 threads leave 128 registers a lane
        qmm_small_kernel<LOWBIT_BITS, NT, 16, MR><<<grid, dim3(1024), 0, s>>>(p);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_small_nt(const QmmParams& p, int waves, hipStream_t s) {
  if (p.M <= 4) return launch_small_mr<NT, 1>(p, waves, s);
  if (p.M <= 8) return launch_small_mr<NT, 2>(p, waves, s);
  return launch_small_mr<NT, 4>(p, waves, s);
}

#define LOWBIT_CAT2(a, b) a##b
#define LOWBIT_CAT(a, b) LOWBIT_CAT2(a, b)
hipError_t LOWBIT_CAT(launch_qmm_b, LOWBIT_BITS)(const QmmParams& p, const QmmLaunch& l, int act,
                                                 hipStream_t s) {
  hipError_t e;
  switch (act) {
    case ACT_F16: e = launch_act<ACT_F16>(p, l, s); break;
    case ACT_BF16: e = LOWBIT_CAT(launch_qmm_bf16_b, LOWBIT_BITS)(p, l, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || l.grid.z == 1) return e;
  auto log2i = [](int v) { int k = 0; while ((1 << k) < v) ++k; return k; };
  QmmReduceShape r{};
  r.splits = static_cast<int>(l.grid.z);
  r.tiles_n = static_cast<int>(l.grid.x);
  r.mtt_shift = log2i(l.mtt);
  r.nt_shift = log2i(l.nt);
  r.wv_shift = log2i(l.waves);
  r.plane_recs = static_cast<int64_t>(l.grid.x) * l.grid.y * l.waves * l.mtt * l.nt * 64;
  const dim3 rgrid(static_cast<unsigned>((r.plane_recs + 255) / 256));
  if (act == ACT_F16) qmm_reduce_kernel<ACT_F16><<<rgrid, dim3(256), 0, s>>>(p, r);
  else qmm_reduce_kernel<ACT_BF16><<<rgrid, dim3(256), 0, s>>>(p, r);
  return hipGetLastError();
}

}  // namespace lowbit

namespace lowbit {
hipError_t LOWBIT_CAT(launch_qmm_small_b, LOWBIT_BITS)(const QmmParams& p, int nt, int waves, hipStream_t s) {
  if (p.M < 1 || p.M > 16) return hipErrorInvalidValue;
  switch (nt) {
    case 1: return launch_small_nt<1>(p, waves, s);
    case 2: return launch_small_nt<2>(p, waves, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace lowbit
