// Linear over int8 activations (the activation-quantized variant: 8-bit
// dynamic activations with groupwise low-bit weights, the export mode that
// "[MPS] Add support for Int4 groupwise quantization" runs with 4-bit weights
// in groups of 32) on the gfx950 int8 MFMA:
//
//   y[m, n] = a_m * sum_g (s[n, g] * P[m, n, g] + z[n, g] * X[m, g]) (+ bias[n])
//   P = sum over group g of xq * q   (exact in int32)
//   X = sum over group g of xq       (exact in int32)
//
// Both integer sums come from v_mfma_i32_16x16x64_i8: P with the codes as
// the B operand, X with a ones operand, so X lands in the same lanes as P
// (with groups of 32, X is computed once per activation fragment by the wave
// that loads it and shared as fp32 through LDS).
// Each group's sums are turned into fp32 and scaled once (two fused
// multiply-adds per output and group), and a_m and the bias enter once at
// the store, rounded once to the output type.
//
// Operand layout: a 64-wide K window per MFMA; lane l supplies row (A) or
// column (B) l % 16 and the 16 K positions 16 (l / 16) .. 16 (l / 16) + 15
// of the window, one byte each, in order.  The MFMA pairs byte e of lane
// group j of A with byte e of lane group j of B, so any fixed assignment of
// K positions to (lane group, byte) that both operands share gives the same
// sums; this one lets A be one 16-byte load of a row and B the 2*BITS bytes
// of 16 consecutive codes.  A group of 32 is half a window: its two groups
// take two passes whose B (and ones) operands are zero in the other half's
// lane groups; a row of K = 64 w + 32 ends with a half window, whose missing
// half the lanes read from the window's first half and mask out.
//
// Block: 4 waves, each NT 16-column tiles over MTT 16-row tiles and all of
// K (the activation operand and its row sums X serve the NT column tiles).
// The operands of 8 / MTT windows are loaded one such batch ahead; the
// activation fragments of a batch, the same for every wave of the block,
// are loaded a quarter per wave and shared through two LDS slabs, one
// barrier per batch (without a memory fence: the code and scale loads of
// the next batch stay in flight).  Every wave runs every barrier: a wave
// past N computes clamped columns and stores nothing.
//
// What bounds it: the vector-memory address unit, not the MFMAs (counters at
// M = 128, K = 4096, N = 14336 with one column tile and one load per scale:
// the address unit busy 82 % of the kernel and stalled on the cache 55 %,
// VALU and MFMA mostly idle).  Every load instruction occupies it about the
// same whatever its width, so the kernel issues few, wide ones: per 16 x 16
// output tile and window about 1/(4 NT) activation loads, 1/MTT code loads
// and (groups of 32) 1/4 scale/zero loads, the scales and zeros of a batch
// coming as one vector per column tile.
#include "qmm_common.h"

#ifndef LOWBIT_BITS
#error "compile with -DLOWBIT_BITS=<1..7>"
#endif

namespace lowbit {

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t mfma_i8(i32x4_t a, i32x4_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// The words holding one lane's 16 codes (K positions kk .. kk + 15 of a
// weight row, kk % 16 == 0): 2*BITS bytes from byte kk*BITS/8.  For even
// BITS they are whole aligned words; for odd BITS they may start in the
// middle of a word, so one more word is read and the lane shifts by 16 bits.
// (The extra bytes belong to the next 16 codes of the same row.)
template <int BITS>
struct CodeWords {
  static constexpr int NL = (BITS + 1) / 2;
  uint32_t w[NL];
  uint32_t sh;
};

template <int BITS>
__device__ __forceinline__ void load_code_words(const uint8_t* row, uint32_t kk,
                                                CodeWords<BITS>& cw) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  constexpr int NL = CodeWords<BITS>::NL;
  const uint32_t off = (kk >> 4) * (2 * BITS);
  const uint8_t* src = static_cast<const uint8_t*>(__builtin_assume_aligned(row + (off & ~3u), 4));
  if constexpr (NL == 1) {
    __builtin_memcpy(&cw.w[0], src, 4);
  } else if constexpr (NL == 2) {
    u32x2 v;
    __builtin_memcpy(&v, src, 8);
    cw.w[0] = v.x; cw.w[1] = v.y;
  } else if constexpr (NL == 3) {
    u32x3 v;
    __builtin_memcpy(&v, src, 12);
    cw.w[0] = v.x; cw.w[1] = v.y; cw.w[2] = v.z;
  } else {
    u32x4 v;
    __builtin_memcpy(&v, src, 16);
    cw.w[0] = v.x; cw.w[1] = v.y; cw.w[2] = v.z; cw.w[3] = v.w;
  }
  cw.sh = (off & 3u) * 8u;
}

// The 16 codes as 16 bytes in K order (the B operand).
template <int BITS>
__device__ __forceinline__ i32x4_t expand_codes(const CodeWords<BITS>& cw) {
  constexpr int NL = CodeWords<BITS>::NL;
  uint32_t S[NL];
  if constexpr (BITS % 2 == 1) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
      S[i] = __builtin_amdgcn_alignbit(i + 1 < NL ? cw.w[i + 1] : 0u, cw.w[i], cw.sh);
  } else {
#pragma unroll
    for (int i = 0; i < NL; ++i) S[i] = cw.w[i];
  }
  if constexpr (BITS == 4) {
    // even codes in the bytes of lo, odd codes in the bytes of hi; two byte
    // permutes per word put them in order
    const uint32_t lo0 = and_nibbles(S[0]), hi0 = and_nibbles(S[0] >> 4);
    const uint32_t lo1 = and_nibbles(S[1]), hi1 = and_nibbles(S[1] >> 4);
    return i32x4_t{static_cast<int>(__builtin_amdgcn_perm(hi0, lo0, 0x05010400u)),
                   static_cast<int>(__builtin_amdgcn_perm(hi0, lo0, 0x07030602u)),
                   static_cast<int>(__builtin_amdgcn_perm(hi1, lo1, 0x05010400u)),
                   static_cast<int>(__builtin_amdgcn_perm(hi1, lo1, 0x07030602u))};
  } else {
    uint32_t d[4];
    static_for<4>([&](auto dd) {
      constexpr int D = decltype(dd)::value;
      d[D] = code_at<BITS, 4 * D>(S) | (code_at<BITS, 4 * D + 1>(S) << 8) |
             (code_at<BITS, 4 * D + 2>(S) << 16) | (code_at<BITS, 4 * D + 3>(S) << 24);
    });
    return i32x4_t{static_cast<int>(d[0]), static_cast<int>(d[1]), static_cast<int>(d[2]),
                   static_cast<int>(d[3])};
  }
}

template <int BITS, int MTT, int NT, bool G32, int SZ>
__global__ __launch_bounds__(256) void qmm_a8_kernel(A8Params p) {
  using T = typename Act<SZ>::bits_t;
  constexpr int TB = static_cast<int>(sizeof(T));
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wv) * 16 * NT;   // waves past N compute clamped columns, store nothing
  const int c = lane & 15;
  const uint32_t j = lane >> 4;
  const int m0 = blockIdx.y * 16 * MTT;
  const uint8_t* wrow[NT];
  const T* srow[NT];
  const T* zrow[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const int nc = min(n0 + 16 * q + c, p.N - 1);
    wrow[q] = p.packed + static_cast<size_t>(nc) * p.row_bytes;
    srow[q] = static_cast<const T*>(p.scales) + static_cast<size_t>(nc) * p.groups;
    zrow[q] = static_cast<const T*>(p.zeros) + static_cast<size_t>(nc) * p.groups;
  }
  const int8_t* arow[MTT];
#pragma unroll
  for (int t = 0; t < MTT; ++t)
    arow[t] = p.xq + static_cast<size_t>(min(m0 + 16 * t + c, p.M - 1)) * p.K;

  const uint32_t K = p.K;
  const int W = static_cast<int>((K + 63) >> 6);
  const int wg_shift = G32 ? 0 : __builtin_ctz(static_cast<uint32_t>(p.group >> 6));
  const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const i32x4_t zero4 = {0, 0, 0, 0};

  // K position of this lane's 16 codes in window w; the missing half of a
  // final half window reads the window's first half (masked out below)
  auto lane_k = [&](int w) -> uint32_t {
    const uint32_t kk = 64u * static_cast<uint32_t>(w) + 16u * j;
    return kk >= K ? kk - 32u : kk;
  };

  // group-32 passes: the lane groups of pass h are 2h and 2h + 1
  const i32x4_t keep0 = (j >> 1) == 0 ? i32x4_t{-1, -1, -1, -1} : zero4;
  const i32x4_t keep1 = (j >> 1) == 1 ? i32x4_t{-1, -1, -1, -1} : zero4;
  const i32x4_t ones0 = ones & keep0, ones1 = ones & keep1;

  // Operands of U consecutive windows (U = 8 / MTT: a batch holds eight
  // activation fragments at every MTT, two per wave), loaded one batch
  // ahead.  The scales and zeros of a batch are kept as raw words, SG values
  // of T per column tile (two per window with groups of 32, else one).
  constexpr int U = 8 / MTT;
  constexpr int SG = G32 ? 2 * U : U;
  constexpr int SZW = (SG * TB + 3) / 4;
  struct Batch {
    CodeWords<BITS> cw[U][NT];
    uint32_t sw[NT][SZW], zw[NT][SZW];
  };
  // The activation fragments of a batch, (window, row tile) f = u * MTT + t,
  // are the same for every wave of the block: each wave loads two of the
  // eight one batch ahead and writes them to one of two LDS slabs, which all
  // four waves read.
  constexpr int NF = U * MTT;   // 8
  static_assert(NF == 8, "two fragments per wave");
  __shared__ i32x4_t s_a[2][NF][64];
  auto load_frags = [&](int bi, i32x4_t (&fr)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = 2 * wv + i, u = f / MTT, t = f % MTT;
      const int w = min(bi * U + u, W - 1);
      fr[i] = *reinterpret_cast<const i32x4_t*>(arow[t] + lane_k(w));
    }
  };
  // Groups of 32: the row sums X of a fragment's two groups (the same for
  // every column) are computed once, by the wave that loads the fragment,
  // and shared as fp32 through LDS: s_x[buf][f][h][j] holds rows 4j .. 4j+3.
  __shared__ float4_t s_x[2][G32 ? NF : 1][2][4];
  auto store_frags = [&](int buf, const i32x4_t (&fr)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) s_a[buf][2 * wv + i][lane] = fr[i];
    if constexpr (G32) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const i32x4_t x = mfma_i8(fr[i], h == 0 ? ones0 : ones1, zero4);
          if (c == 0)
            s_x[buf][2 * wv + i][h][j] = float4_t{static_cast<float>(x[0]), static_cast<float>(x[1]),
                                                  static_cast<float>(x[2]), static_cast<float>(x[3])};
        }
      }
    }
  };
  // LDS writes done, then meet the other waves; no memory fence, so the
  // global loads in flight stay in flight
  auto lds_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); };
  // The scales (and zeros) of a batch are SG consecutive groups of the row,
  // slot i holding group g0 + i (g0: the batch's first group, rounded down
  // to an even group for 2-byte values so that the slots start 4-byte
  // aligned); they come in one vector load per column tile when the slots
  // lie inside the row and the rows are 4-byte aligned (every load
  // instruction costs the address unit about the same, whatever its width),
  // otherwise one load per group.
  const bool sz_wide = (TB == 4 || (p.groups % 2 == 0)) &&
                       ((reinterpret_cast<uintptr_t>(p.scales) | reinterpret_cast<uintptr_t>(p.zeros)) & 3u) == 0;
  auto batch_g0 = [&](int bi) -> int {
    if constexpr (G32) return SG * bi;
    else return TB == 2 ? ((bi * U) >> wg_shift) & ~1 : ((bi * U) >> wg_shift);
  };
  auto load_words = [&](const T* src, uint32_t (&wd)[SZW]) {
    const uint32_t* s4 = static_cast<const uint32_t*>(__builtin_assume_aligned(src, 4));
    if constexpr (SZW % 4 == 0) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < SZW / 4; ++q) {
        u32x4 v;
        __builtin_memcpy(&v, s4 + 4 * q, 16);
        wd[4 * q] = v.x; wd[4 * q + 1] = v.y; wd[4 * q + 2] = v.z; wd[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < SZW; ++q) wd[q] = s4[q];
    }
  };
  auto load_batch = [&](int bi, Batch& bt) {
    const int g0 = batch_g0(bi);
    const bool wide = sz_wide && g0 + SG <= p.groups;
    if (wide) {
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        load_words(srow[q] + g0, bt.sw[q]);
        load_words(zrow[q] + g0, bt.zw[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NT; ++q) {
#pragma unroll
        for (int i = 0; i < SZW; ++i) {
          bt.sw[q][i] = 0u;
          bt.zw[q][i] = 0u;
        }
#pragma unroll
        for (int g = 0; g < SG; ++g) {
          const int idx = min(g0 + g, p.groups - 1);
          const uint32_t sh = 8u * static_cast<uint32_t>((g * TB) % 4);
          bt.sw[q][(g * TB) / 4] |= static_cast<uint32_t>(srow[q][idx]) << sh;
          bt.zw[q][(g * TB) / 4] |= static_cast<uint32_t>(zrow[q][idx]) << sh;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = min(bi * U + u, W - 1);
      const uint32_t kk = lane_k(w);
#pragma unroll
      for (int q = 0; q < NT; ++q) load_code_words<BITS>(wrow[q], kk, bt.cw[u][q]);
    }
  };
  // slot g (0 .. SG-1) of a batch's raw words, as fp32: g a compile-time
  // constant (groups of 32), or (groups of 64 and more) a wave-uniform index
  // known only at run time, picked by selects over the slots (an array
  // indexed at run time would live in scratch)
  auto sz_slot = [&](const uint32_t (&wd)[SZW], int i) -> float {
    if constexpr (TB == 4) return __uint_as_float(wd[i]);
    else return act_bits_to_float<SZ>((wd[i >> 1] >> (16 * (i & 1))) & 0xffffu);
  };
  auto sz_value = [&](const uint32_t (&wd)[SZW], int g) -> float {
    if constexpr (G32) {
      return sz_slot(wd, g);
    } else {
      // (each slot made opaque first: a select chain over plain array
      // elements would be folded back into an indexed access)
      float v = sz_slot(wd, 0);
#pragma unroll
      for (int i = 1; i < SG; ++i) {
        float t = sz_slot(wd, i);
        asm("" : "+v"(t));
        v = g == i ? t : v;
      }
      return v;
    }
  };


  float acc[MTT][NT][4];
  i32x4_t P[MTT][NT], X[MTT];
#pragma unroll
  for (int t = 0; t < MTT; ++t) {
    X[t] = zero4;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      P[t][q] = zero4;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][q][i] = 0.0f;
    }
  }
  // acc += s * P + z * X for every tile (X as fp32: from LDS with groups of
  // 32, else converted here once per row tile)
  auto rescale = [&](const Batch& bt, int g, int buf, int u, int h) {
#pragma unroll
    for (int t = 0; t < MTT; ++t) {
      float xf[4];
      if constexpr (G32) {
        const float4_t xv = s_x[buf][u * MTT + t][h][j];
        xf[0] = xv[0]; xf[1] = xv[1]; xf[2] = xv[2]; xf[3] = xv[3];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xf[i] = static_cast<float>(X[t][i]);
      }
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const float sv = sz_value(bt.sw[q], g), zv = sz_value(bt.zw[q], g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[t][q][i] = fmaf(sv, static_cast<float>(P[t][q][i]), acc[t][q][i]);
          acc[t][q][i] = fmaf(zv, xf[i], acc[t][q][i]);
        }
      }
    }
  };

  const int NB = (W + U - 1) / U;
  Batch cur;
  i32x4_t fr[2];
  load_frags(0, fr);
  load_batch(0, cur);
  store_frags(0, fr);
  lds_barrier();
  load_frags(min(1, NB - 1), fr);
  for (int bi = 0; bi < NB; ++bi) {
    const int buf = bi & 1;
    Batch nxt;
    load_batch(min(bi + 1, NB - 1), nxt);   // the last batch loads itself again
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = bi * U + u;
      if (w >= W) break;
      i32x4_t b[NT];
#pragma unroll
      for (int q = 0; q < NT; ++q) b[q] = expand_codes<BITS>(cur.cw[u][q]);
      if constexpr (G32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && 64u * static_cast<uint32_t>(w) + 64u > K) break;   // a half window
          const i32x4_t keep = h == 0 ? keep0 : keep1;
#pragma unroll
          for (int t = 0; t < MTT; ++t) {
            const i32x4_t at = s_a[buf][u * MTT + t][lane];
#pragma unroll
            for (int q = 0; q < NT; ++q) P[t][q] = mfma_i8(at, b[q] & keep, zero4);
          }
          rescale(cur, 2 * u + h, buf, u, h);
        }
      } else {
#pragma unroll
        for (int t = 0; t < MTT; ++t) {
          const i32x4_t at = s_a[buf][u * MTT + t][lane];
          X[t] = mfma_i8(at, ones, X[t]);
#pragma unroll
          for (int q = 0; q < NT; ++q) P[t][q] = mfma_i8(at, b[q], P[t][q]);
        }
        if (((w + 1) & ((1 << wg_shift) - 1)) == 0) {   // last window of its group
          rescale(cur, (w >> wg_shift) - batch_g0(bi), buf, u, 0);
#pragma unroll
          for (int t = 0; t < MTT; ++t) {
            X[t] = zero4;
#pragma unroll
            for (int q = 0; q < NT; ++q) P[t][q] = zero4;
          }
        }
      }
    }
    cur = nxt;
    // the next batch's fragments into the other slab (last read one batch
    // ago, before the previous barrier), then the one after that in flight
    store_frags(buf ^ 1, fr);
    lds_barrier();
    load_frags(min(bi + 2, NB - 1), fr);
  }

  // D layout of a 16x16 MFMA tile: lane l holds rows 4 (l / 16) + i of column l % 16
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const int n = n0 + 16 * q + c;
    if (n >= p.N) break;
    const float bias = p.bias ? act_bits_to_float<SZ>(static_cast<const T*>(p.bias)[n]) : 0.0f;
#pragma unroll
    for (int t = 0; t < MTT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * t + 4 * static_cast<int>(j) + i;
        if (m < p.M)
          store_act<SZ>(p.y, static_cast<size_t>(m) * p.N + n, fmaf(p.ascale[m], acc[t][q][i], bias));
      }
    }
  }
}

// (The launch helpers carry BITS: every width is compiled into its own
// object, and helpers without it would be one symbol with seven bodies.)
template <int BITS, int MTT, int NT, bool G32, int SZ>
hipError_t launch_a8(const A8Params& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.N + 64 * NT - 1) / (64 * NT)),
                  static_cast<unsigned>((p.M + 16 * MTT - 1) / (16 * MTT)));
  qmm_a8_kernel<BITS, MTT, NT, G32, SZ><<<grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <int BITS, int MTT, int NT, bool G32>
hipError_t launch_a8_sz(const A8Params& p, int sz, hipStream_t s) {
  switch (sz) {
    case ACT_F32: return launch_a8<BITS, MTT, NT, G32, ACT_F32>(p, s);
    case ACT_F16: return launch_a8<BITS, MTT, NT, G32, ACT_F16>(p, s);
    default: return launch_a8<BITS, MTT, NT, G32, ACT_BF16>(p, s);
  }
}

template <int BITS, int MTT, int NT>
hipError_t launch_a8_g(const A8Params& p, int sz, hipStream_t s) {
  return p.group == 32 ? launch_a8_sz<BITS, MTT, NT, true>(p, sz, s)
                       : launch_a8_sz<BITS, MTT, NT, false>(p, sz, s);
}

#define LOWBIT_CAT2(a, b) a##b
#define LOWBIT_CAT(a, b) LOWBIT_CAT2(a, b)
hipError_t LOWBIT_CAT(launch_qmm_a8_b, LOWBIT_BITS)(const A8Params& p, int mtt, int nt, int sz,
                                                   hipStream_t s) {
  if (nt == 2) {
    switch (mtt) {
      case 1: return launch_a8_g<LOWBIT_BITS, 1, 2>(p, sz, s);
      case 2: return launch_a8_g<LOWBIT_BITS, 2, 2>(p, sz, s);
      default: return launch_a8_g<LOWBIT_BITS, 4, 2>(p, sz, s);
    }
  }
  switch (mtt) {
    case 1: return launch_a8_g<LOWBIT_BITS, 1, 1>(p, sz, s);
    case 2: return launch_a8_g<LOWBIT_BITS, 2, 1>(p, sz, s);
    default: return launch_a8_g<LOWBIT_BITS, 4, 1>(p, sz, s);
  }
}

}  // namespace lowbit
