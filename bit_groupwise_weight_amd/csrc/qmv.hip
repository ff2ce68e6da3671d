// Decode matrix-vector kernel (small M): y = x . dequant(Wq)^T (+ bias).
//
// Prior art: the qmv_fast Metal kernel of "metal lowbit kernels: qmv_fast
// optimization" (Summary) streams packed rows and applies the N x num_groups
// scales and zeros inside the dot product.  This kernel keeps that idea and is
// laid out for CDNA4:
//   * a row's codes are cut into 32-code runs; a run of b-bit codes is
//     exactly b 32-bit words, fetched with one or two vector loads;
//   * 2^lpr_shift lanes of a wavefront share a group of R rows; in round t
//     lane l owns runs 4*t*lanes + l + lanes*j (j = 0..3) of each of its R
//     rows, so that each load instruction of the group reads one contiguous
//     span of the packed row;
//   * the block stages the activations of the round once in LDS, already
//     rearranged into the operand pairs the unpack plan needs, together with
//     each 32-code run's activation sum X; activation
//     loads are issued before the weight loads so the stage is ready while the
//     weights are still in flight;
//   * codes reach the dot products as exact values: fp16 codes as fp16
//     subnormals q * 2^(o-24), two per 32-bit word at one bit offset o of
//     their halves (funnel-shift windows or byte permutes, qmv_plan.h),
//     masked with one AND and multiplied with one v_dot2_f32_f16, one fp32
//     accumulator per offset; bf16 codes through the fp8 conversion (a code
//     below 16 in a byte is the e4m3 value q * 2^-9) or, above 4 bits,
//     through fp32; fp32 converts each code.  Only the products x*q enter
//     the fp32 sums, so their rounding is relative to sum |x*q|;
//   * per 32-code run (which never crosses a group):
//       y += s * (sum_k x_k q_k) + z * X;
//   * the R row partial sums of the lanes of a row group are combined with
//     DPP lane moves; bias is added in fp32 and the result rounded once.
#include "device_common.h"
#include "kernels.h"
#include "qmv_plan.h"

#ifndef LOWBIT_BITS
#error "compile with -DLOWBIT_BITS=<1..7>"
#endif

namespace lowbit {

// Units of the per-row sums until the store: fp16 runs keep their products
// in the units of the subnormal codes, 2^-24 (x * q * 2^-24 exactly), so the
// run sums P and X are both taken in those units (X from dot2 with the
// smallest fp16 subnormal, 2^-24, as the weight of each activation) and the
// row sum is scaled by 2^24 once, at the store.  bf16 and fp32: units of 1.
template <int ACT> struct SumUnit {
  static constexpr uint32_t xweight = Magic<ACT>::ones;   // (unused for fp32)
  static constexpr float to_one = 1.0f;
};
template <> struct SumUnit<ACT_F16> {
  static constexpr uint32_t xweight = 0x00010001u;        // 2^-24 in each half
  static constexpr float to_one = 16777216.0f;            // 2^24
};

// Raw activation words per 32-code run and staged words per run.
template <int ACT> struct RawWords { static constexpr int n = (ACT == ACT_F32) ? 32 : 16; };
template <int ACT, int BITS> struct StagedWords;
template <int BITS> struct StagedWords<ACT_F16, BITS> { static constexpr int n = F16Slots<BITS>::n; };
template <int BITS> struct StagedWords<ACT_BF16, BITS> { static constexpr int n = 16; };
template <int BITS> struct StagedWords<ACT_F32, BITS> { static constexpr int n = 32; };
// uint4 quads per staged run: the words, then X, padded to 16 bytes.
template <int ACT, int BITS> struct RunQuads {
  static constexpr int n = (StagedWords<ACT, BITS>::n + 1 + 3) / 4;
};

// ---------------------------------------------------------------- staging --

// Slot I's activation pair: x[klo] in the low half, x[khi] in the high half,
// gathered from the raw pairs (x[2i], x[2i+1]) with one byte permute (a
// missing code's half selects zero bytes).
template <int BITS, int I = 0>
__device__ __forceinline__ void f16_stage_slots(const uint32_t* raw, uint32_t* out) {
  if constexpr (I < F16Slots<BITS>::n) {
    constexpr int klo = F16Slots<BITS>::klo(I), khi = F16Slots<BITS>::khi(I);
    constexpr uint32_t kZero = 0x0cu;   // v_perm_b32 selector of a zero byte
    constexpr uint32_t lo0 = klo >= 0 ? (klo & 1) * 2u : kZero;       // bytes of S1
    constexpr uint32_t hi0 = khi >= 0 ? 4u + (khi & 1) * 2u : kZero;  // bytes of S0
    constexpr uint32_t sel = lo0 | ((klo >= 0 ? lo0 + 1 : kZero) << 8) | (hi0 << 16) |
                             ((khi >= 0 ? hi0 + 1 : kZero) << 24);
    out[I] = __builtin_amdgcn_perm(raw[(khi >= 0 ? khi : 0) >> 1], raw[(klo >= 0 ? klo : 0) >> 1], sel);
    f16_stage_slots<BITS, I + 1>(raw, out);
  }
}

// Turn 32 raw activations into the staged words of one run (+ X).
template <int ACT, int BITS>
__device__ __forceinline__ void stage_run(const uint32_t* raw, uint32_t* out) {
  constexpr int W = StagedWords<ACT, BITS>::n;
  float X = 0.0f;
  if constexpr (ACT == ACT_F32) {
#pragma unroll
    for (int i = 0; i < 32; ++i) { out[i] = raw[i]; X += __uint_as_float(raw[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) X = dot2<ACT>(raw[i], SumUnit<ACT>::xweight, X);
    if constexpr (ACT == ACT_F16) {
      f16_stage_slots<BITS>(raw, out);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = raw[i];
    }
  }
  out[W] = __float_as_uint(X);
#pragma unroll
  for (int i = W + 1; i < RunQuads<ACT, BITS>::n * 4; ++i) out[i] = 0u;
}

// ------------------------------------------------------------------ dots --

// Bits [Q, Q + 32) of the run's code stream (zero past its end).
template <int BITS, int Q>
__device__ __forceinline__ uint32_t stream_word(const uint32_t* w) {
  constexpr int d = Q / 32, sh = Q % 32;
  if constexpr (d >= BITS) return 0u;
  else if constexpr (sh == 0) return w[d];
  else if constexpr (d + 1 < BITS) return __builtin_amdgcn_alignbit(w[d + 1], w[d], sh);
  else return w[d] >> sh;
}

// fp16: slot I of the plan (qmv_plan.h) as one word holding its two codes
// at bit offset F16Slots<BITS>::offset(I) of their halves, every other bit
// clear: the halves read as the fp16 subnormals q * 2^(o-24).
template <int BITS, int I>
constexpr int f16_slot_offset() {
  if constexpr (16 % BITS == 0) {
    constexpr PairSlot s = F16Slots<BITS>::Plan::table.s[I];
    static_assert(s.klo < 0 || s.khi < 0 || s.olo == s.ohi, "paired codes share their offset");
  }
  return F16Slots<BITS>::offset(I);
}

template <int BITS, int I>
__device__ __forceinline__ uint32_t f16_slot_word(const uint32_t* w) {
  constexpr uint32_t m = (1u << BITS) - 1u;
  if constexpr (16 % BITS == 0) {
    // funnel-shift window of word s.word
    constexpr PairSlot s = F16Slots<BITS>::Plan::table.s[I];
    constexpr uint32_t mask = (s.klo >= 0 ? (m << s.olo) : 0u) |
                              (s.khi >= 0 ? (m << (16 + s.ohi)) : 0u);
    return stream_word<BITS, 32 * s.word + s.shift>(w) & mask;
  } else {
    // two halves gathered by one byte permute
    constexpr PermSlot s = F16PermPlan<BITS>::table.s[I];
    static_assert(s.o >= 0 && s.o + BITS <= 11, "the code stays below bit 11 of its half");
    constexpr uint32_t mask = (m << s.o) | (m << (16 + s.o));
    return __builtin_amdgcn_perm(stream_word<BITS, s.q0>(w), stream_word<BITS, s.q1>(w), s.sel) &
           mask;
  }
}

// Slots visited by offset, highest first, so that one accumulator serves all
// of them: before the slots of a lower offset the running sum is scaled by
// the (exact) power of two between the two offsets, which keeps it equal to
// sum x*q * 2^(o-24) at the current offset o (Horner).
struct SlotOrder {
  int idx[32];
  int n;
};

template <int BITS>
constexpr SlotOrder f16_slot_order() {
  SlotOrder ord{};
  ord.n = F16Slots<BITS>::n;
  int j = 0;
  for (int o = 10; o >= 0; --o)
    for (int i = 0; i < ord.n; ++i)
      if (F16Slots<BITS>::offset(i) == o) ord.idx[j++] = i;
  return ord;
}

template <int BITS, int J>
__device__ __forceinline__ float f16_chain(const uint32_t* w, const uint32_t* xs, float t) {
  constexpr SlotOrder ord = f16_slot_order<BITS>();
  if constexpr (J < ord.n) {
    constexpr int I = ord.idx[J];
    constexpr int o = f16_slot_offset<BITS, I>();
    if constexpr (J > 0) {
      constexpr int prev = f16_slot_offset<BITS, ord.idx[J - 1]>();
      if constexpr (prev != o) t *= 1.0f / static_cast<float>(1u << (prev - o));
    }
    t = dot2<ACT_F16>(xs[I], f16_slot_word<BITS, I>(w), t);
    return f16_chain<BITS, J + 1>(w, xs, t);
  } else {
    return t;
  }
}

// sum_k x_k q_k * 2^-24 over one fp16 run: the chain ends at the lowest
// offset, which every plan has at 0.
template <int BITS>
__device__ __forceinline__ float f16_run_dot(const uint32_t* w, const uint32_t* xs) {
  constexpr SlotOrder ord = f16_slot_order<BITS>();
  static_assert(f16_slot_offset<BITS, ord.idx[ord.n - 1]>() == 0, "chain ends at offset 0");
  return f16_chain<BITS, 0>(w, xs, 0.0f);
}

// Codes 2I and 2I+1 of a run as two exact bf16 values (low half: code 2I).
// Up to 4 bits, a code q in a byte is the OCP fp8 e4m3 value q * 2^-9 (a
// subnormal below 8, then the first binade with step 2^-9), so one scaled
// fp8 conversion by 2^9 gives both; wider codes go through fp32, where the
// bf16 value is the top half of the fp32 one (exact for q < 256).
template <int BITS, int I>
__device__ __forceinline__ uint32_t bf16_code_pair(const uint32_t* w) {
  if constexpr (BITS <= 4) {
    const uint32_t b = code_at<BITS, 2 * I>(w) | (code_at<BITS, 2 * I + 1>(w) << 8);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 512.0f, false));
  } else {
    const uint32_t f0 = __float_as_uint(static_cast<float>(code_at<BITS, 2 * I>(w)));
    const uint32_t f1 = __float_as_uint(static_cast<float>(code_at<BITS, 2 * I + 1>(w)));
    return __builtin_amdgcn_perm(f1, f0, 0x07060302u);
  }
}

template <int BITS, int I = 0>
__device__ __forceinline__ float bf16_dot_pairs(const uint32_t* w, const uint32_t* xs, float acc) {
  if constexpr (I < 16) {
    acc = dot2<ACT_BF16>(xs[I], bf16_code_pair<BITS, I>(w), acc);
    return bf16_dot_pairs<BITS, I + 1>(w, xs, acc);
  } else {
    return acc;
  }
}

template <int BITS, int I = 0>
__device__ __forceinline__ float f32_dot(const uint32_t* w, const uint32_t* xs, float acc) {
  if constexpr (I < 32) {
    acc = __builtin_fmaf(__uint_as_float(xs[I]), static_cast<float>(code_at<BITS, I>(w)), acc);
    return f32_dot<BITS, I + 1>(w, xs, acc);
  } else {
    return acc;
  }
}

// Widths dividing 8: byte planes.  Plane j of a word keeps bits j*b.. of
// every byte, i.e. code CPB*i + j of the word in byte i (CPB = 8/b codes per
// byte), so one shift and one AND serve four codes and each code converts with
// one v_cvt_f32_ubyteN (instead of a field extract and a conversion).
template <int BITS>
__device__ __forceinline__ float f32_dot_planes(const uint32_t* w, const uint32_t* xs) {
  constexpr int CPB = 8 / BITS;
  constexpr int CPW = 32 / BITS;                   // codes per word
  constexpr uint32_t m = ((1u << BITS) - 1u) * 0x01010101u;
  float acc = 0.0f;
#pragma unroll
  for (int d = 0; d < BITS; ++d) {
#pragma unroll
    for (int j = 0; j < CPB; ++j) {
      uint32_t plane = (w[d] >> (j * BITS)) & m;
      asm("" : "+v"(plane));   // (opaque: else the byte reads fold back into field extracts)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = d * CPW + i * CPB + j;
        acc = __builtin_fmaf(__uint_as_float(xs[k]), static_cast<float>((plane >> (8 * i)) & 0xffu), acc);
      }
    }
  }
  return acc;
}

// sum_k x_k q_k over one run (in SumUnit<ACT> units), from the staged words
// and the run's code words.
template <int ACT, int BITS>
__device__ __forceinline__ float run_dot(const uint32_t* w, const uint32_t* xs) {
  if constexpr (ACT == ACT_F16) {
    return f16_run_dot<BITS>(w, xs);
  } else if constexpr (ACT == ACT_BF16) {
    return bf16_dot_pairs<BITS>(w, xs, 0.0f);
  } else if constexpr (8 % BITS == 0) {
    return f32_dot_planes<BITS>(w, xs);
  } else {
    return f32_dot<BITS>(w, xs, 0.0f);
  }
}

// ----------------------------------------------------------------- loads --

// The BITS words of one 32-code run (4-byte aligned): one vector load for
// BITS <= 4, two above.
template <int BITS>
__device__ __forceinline__ void load_run(const uint8_t* src, uint32_t* w) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const uint8_t* s = static_cast<const uint8_t*>(__builtin_assume_aligned(src, 4));
  constexpr int O = BITS >= 4 ? 4 : 0;
  constexpr int REST = BITS - O;
  if constexpr (BITS >= 4) {
    u32x4 v;
    __builtin_memcpy(&v, s, 16);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  if constexpr (REST == 3) {
    u32x3 v;
    __builtin_memcpy(&v, s + 4 * O, 12);
    w[O] = v.x; w[O + 1] = v.y; w[O + 2] = v.z;
  } else if constexpr (REST == 2) {
    u32x2 v;
    __builtin_memcpy(&v, s + 4 * O, 8);
    w[O] = v.x; w[O + 1] = v.y;
  } else if constexpr (REST == 1) {
    __builtin_memcpy(&w[O], s + 4 * O, 4);
  }
}

template <int ACT>
__device__ __forceinline__ void load_raw_run(const void* x, int64_t off,
                                             uint32_t (&raw)[RawWords<ACT>::n]) {
  constexpr int Q = RawWords<ACT>::n / 4;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) +
                                                    off * Act<ACT>::bytes);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint4 v = src[q];
    raw[4 * q + 0] = v.x; raw[4 * q + 1] = v.y; raw[4 * q + 2] = v.z; raw[4 * q + 3] = v.w;
  }
}

// Decode kernel: rows are processed by groups of `lanes` lanes (a power of
// two <= 64); each lane takes four 32-code runs of the row per round.  Runs
// are dealt out interleaved -- in round t, slot j of lane l is run
// 4*t*lanes + l + lanes*j -- so that every weight load instruction of a
// row group reads one contiguous span of the packed row.  Each lane
// accumulates, per run, P = sum x*q against activations staged in LDS in the
// form its bit width needs, then y += s*P + z*X (X = sum of the run's x).
template <int BITS, int GROUP, int ACT, int MT, int VAR>
__device__ __forceinline__ void qmv_block(const QmvParams& p, const int bx, uint4* stage) {
  constexpr int R = qmv_rows_per_group(BITS, MT, VAR);   // rows per row group
  constexpr int RAW = RawWords<ACT>::n;
  constexpr int QD = RunQuads<ACT, BITS>::n;    // staged quads per run
  constexpr int GSHIFT = GROUP == 32 ? 5 : GROUP == 64 ? 6 : GROUP == 128 ? 7 : 8;
  constexpr int SQ = qmv_stage_quads_per_lane(MT, QD);   // LDS quads per lane in a group

  const int tid = threadIdx.x;
  const int lanes = 1 << p.lpr_shift;
  const int lane = tid & (lanes - 1);
  const int rg = tid >> p.lpr_shift;
  const int rgs = blockDim.x >> p.lpr_shift;
  const int n_base = (bx * rgs + rg) * R;
  const int m0 = blockIdx.y * MT;
  const int mcount = min(MT, p.M - m0);
  const int nruns = MT * 4 * lanes;              // staged runs per round
  const int runs = p.K >> 5;                     // 32-code runs per row
  const int rounds = (runs + 4 * lanes - 1) >> (p.lpr_shift + 2);

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  for (int t = 0; t < rounds; ++t) {
    const int rbase = 4 * t * lanes;             // first run of the round
    // -- activation loads for this thread's first staged run (issued first).
    // Staged run rr: activation row m, slot j, lane-in-group ul.
    auto run_coords = [&](int rr, int& m, int& ul, int& j) {
      m = rr >> (p.lpr_shift + 2);
      const int rem = rr - (m << (p.lpr_shift + 2));
      ul = rem & (lanes - 1);
      j = rem >> p.lpr_shift;
    };
    auto run_load = [&](int rr, uint32_t (&raw)[RAW]) {
      int m, ul, j;
      run_coords(rr, m, ul, j);
      const int k = (rbase + ul + lanes * j) * 32;
      const bool valid = rr < nruns && m < mcount && k < p.K;
      // (threads without a real run load nothing: at one activation row
      // they are half the block, and their loads would add half again to the
      // block's activation traffic; an invalid run stages zeros)
      if (valid) load_raw_run<ACT>(p.x, static_cast<int64_t>(m0 + m) * p.K + k, raw);
      return valid;
    };
    uint32_t raw[RAW];
    const bool raw_valid = run_load(tid, raw);
    // keep the activation loads ahead of the weight loads: staging then waits
    // only for them, while the weights are still in flight
    __builtin_amdgcn_sched_barrier(0);

    // -- weights, scales and zeros of this lane's four runs (addresses
    // clamped to the matrix: a run past K reads the row's last run, a row
    // past N the last row).  Scales and zeros stay raw bits until first use,
    // so these loads never force an early wait.
    uint32_t d[R][4 * BITS];
    uint32_t sb[R][4], zb[R][4];
    using T = typename Act<ACT>::bits_t;
    // (run and group indices are unsigned 32-bit, so each address is one
    // 64-bit add of a zero-extended offset to a per-row base)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int nc = min(n_base + r, p.N - 1);
      const uint8_t* rowp = p.packed + static_cast<int64_t>(nc) * p.row_bytes;
      const T* srow = static_cast<const T*>(p.scales) + static_cast<int64_t>(nc) * p.groups;
      const T* zrow = static_cast<const T*>(p.zeros) + static_cast<int64_t>(nc) * p.groups;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t run = static_cast<uint32_t>(min(rbase + lane + lanes * j, runs - 1));
        load_run<BITS>(rowp + run * (4u * BITS), &d[r][j * BITS]);
        const uint32_t gi = run >> (GSHIFT - 5);
        sb[r][j] = srow[gi];
        zb[r][j] = zrow[gi];
      }
    }

    // -- stage the round's activations: layout [lane-in-group][m][j][quad],
    // SQ quads per lane (an odd count, so that 16 lanes reading the same
    // quad of their own runs hit 16 distinct 4-bank groups), which makes every
    // read offset below a constant.  The thread's first run (loaded above,
    // before the weights) is staged outside the loop so that only the
    // activation loads must have landed.  Threads without a run (past nruns:
    // at one activation row, half the block) skip the staging arithmetic;
    // runs past M or K stage zeros.
    auto stage_store = [&](int rr, bool valid) {
      int m, ul, j;
      run_coords(rr, m, ul, j);
      uint4* dst = stage + ul * SQ + (m * 4 + j) * QD;
      if (valid) {
        uint32_t out[QD * 4];
        stage_run<ACT, BITS>(raw, out);
#pragma unroll
        for (int q = 0; q < QD; ++q)
          dst[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
      } else {
#pragma unroll
        for (int q = 0; q < QD; ++q) dst[q] = make_uint4(0u, 0u, 0u, 0u);
      }
    };
    if (tid < nruns) stage_store(tid, raw_valid);
    for (int rr = tid + blockDim.x; rr < nruns; rr += blockDim.x) {
      const bool v = run_load(rr, raw);
      stage_store(rr, v);
    }
    __syncthreads();

    // -- compute.  Runs past K have zero staged activations and X = 0, so
    // their clamped copies add s * 0 + z * 0 = 0; rows past N are never
    // stored; activation rows past M are zero and never stored.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint32_t xs[QD * 4];
#pragma unroll
        for (int q = 0; q < QD; ++q) {
          const uint4 v = stage[lane * SQ + (m * 4 + j) * QD + q];
          xs[4 * q] = v.x; xs[4 * q + 1] = v.y; xs[4 * q + 2] = v.z; xs[4 * q + 3] = v.w;
        }
        const float X = __uint_as_float(xs[StagedWords<ACT, BITS>::n]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float dq = run_dot<ACT, BITS>(&d[r][j * BITS], xs);
          const float sv = act_bits_to_float<ACT>(sb[r][j]);
          const float zv = act_bits_to_float<ACT>(zb[r][j]);
          acc[r][m] = __builtin_fmaf(sv, dq, acc[r][m]);
          acc[r][m] = __builtin_fmaf(zv, X, acc[r][m]);
        }
        // With several activation rows, keep one staged fragment live at a
        // time (hoisting them all would take MT*4*QD*4 registers): the empty
        // asm consumes this fragment's sums and, as a memory clobber, keeps
        // the next fragment's LDS reads behind them.  With one row this is
        // the lean variants: fewer registers, one more wave per SIMD, which
        // pays when there are many blocks per CU to overlap.
        if constexpr (MT > 1 || VAR != QMV_DEFAULT) {
#pragma unroll
          for (int r = 0; r < R; ++r) asm volatile("" : "+v"(acc[r][m]) : : "memory");
        }
      }
    }
    if (t + 1 < rounds) __syncthreads();
  }

  // combine the lanes of each row group with DPP; the sum lands in the
  // group's last lane
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = group_sum_to_last(acc[r][m], lanes);
  if (lane == lanes - 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n_base + r;
      if (n >= p.N) continue;
      const float b = p.bias ? load_act<ACT>(p.bias, n) : 0.0f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= mcount) break;
        store_act<ACT>(p.y, static_cast<int64_t>(m0 + m) * p.N + n,
                        __builtin_fmaf(acc[r][m], SumUnit<ACT>::to_one, b));
      }
    }
  }
}

// One problem per launch (its parameters at fixed kernel-argument offsets).
template <int BITS, int GROUP, int ACT, int MT, int VAR>
__global__ __launch_bounds__(256) void qmv_kernel(QmvParams p) {
  extern __shared__ uint4 stage[];
  qmv_block<BITS, GROUP, ACT, MT, VAR>(p, static_cast<int>(blockIdx.x), stage);
}

// Several problems per launch: blockIdx.z selects the problem (no memory
// access needed to find it); blocks past that problem's rows exit at once.
template <int BITS, int GROUP, int ACT, int MT, int VAR>
__global__ __launch_bounds__(256) void qmv_multi_kernel(QmvBatch b) {
  extern __shared__ uint4 stage[];
  const QmvParams& p = b.prob[blockIdx.z];
  const int rows_per_block = (static_cast<int>(blockDim.x) >> p.lpr_shift) * qmv_rows_per_group(BITS, MT, VAR);
  if (static_cast<int>(blockIdx.x) * rows_per_block >= p.N) return;   // block-uniform
  qmv_block<BITS, GROUP, ACT, MT, VAR>(p, static_cast<int>(blockIdx.x), stage);
}

template <int GROUP, int ACT, int MT, int VAR>
static hipError_t launch_one(const QmvBatch& b, const QmvLaunch& l, hipStream_t s) {
  // staged runs (sized for the widest lane group)
  int shift = 0;
  for (unsigned i = 0; i < l.grid.z; ++i) shift = b.prob[i].lpr_shift > shift ? b.prob[i].lpr_shift : shift;
  const size_t lds = (size_t(1) << shift) *
                    qmv_stage_quads_per_lane(MT, RunQuads<ACT, LOWBIT_BITS>::n) * 16;
  if (l.grid.z == 1)
    qmv_kernel<LOWBIT_BITS, GROUP, ACT, MT, VAR><<<l.grid, l.block, lds, s>>>(b.prob[0]);
  else
    qmv_multi_kernel<LOWBIT_BITS, GROUP, ACT, MT, VAR><<<l.grid, l.block, lds, s>>>(b);
  return hipGetLastError();
}

template <int GROUP, int ACT>
static hipError_t dispatch_mt(const QmvBatch& p, const QmvLaunch& l, hipStream_t s) {
  switch (l.mt) {
    case 1:
      // (LEAN2 is LEAN where the default already has two rows per group,
      // LEAN1 is LEAN where it has one)
      if (l.variant == QMV_LEAN2 && qmv_rows_per_group(LOWBIT_BITS, 1, QMV_DEFAULT) == 1)
        return launch_one<GROUP, ACT, 1, QMV_LEAN2>(p, l, s);
      if (l.variant == QMV_LEAN1 && qmv_rows_per_group(LOWBIT_BITS, 1, QMV_DEFAULT) == 2)
        return launch_one<GROUP, ACT, 1, QMV_LEAN1>(p, l, s);
      if (l.variant != QMV_DEFAULT) return launch_one<GROUP, ACT, 1, QMV_LEAN>(p, l, s);
      return launch_one<GROUP, ACT, 1, QMV_DEFAULT>(p, l, s);
    case 2: return launch_one<GROUP, ACT, 2, QMV_LEAN>(p, l, s);
    case 4: return launch_one<GROUP, ACT, 4, QMV_LEAN>(p, l, s);
    default: return hipErrorInvalidValue;
  }
}

template <int GROUP>
static hipError_t dispatch_act(const QmvBatch& p, const QmvLaunch& l, int act, hipStream_t s) {
  switch (act) {
    case ACT_F32: return dispatch_mt<GROUP, ACT_F32>(p, l, s);
    case ACT_F16: return dispatch_mt<GROUP, ACT_F16>(p, l, s);
    case ACT_BF16: return dispatch_mt<GROUP, ACT_BF16>(p, l, s);
    default: return hipErrorInvalidValue;
  }
}

#define LOWBIT_CAT2(a, b) a##b
#define LOWBIT_CAT(a, b) LOWBIT_CAT2(a, b)
hipError_t LOWBIT_CAT(launch_qmv_b, LOWBIT_BITS)(const QmvBatch& p, const QmvLaunch& l,
                                                 int group, int act, hipStream_t s) {
  switch (group) {
    case 32: return dispatch_act<32>(p, l, act, s);
    case 64: return dispatch_act<64>(p, l, act, s);
    case 128: return dispatch_act<128>(p, l, act, s);
    case 256: return dispatch_act<256>(p, l, act, s);
    default: return hipErrorInvalidValue;
  }
}

// Staged LDS bytes per activation row and per four-run slot group of a lane
// in a round (host-side sizing).
#define LOWBIT_QMV_STAGE(ACTK) (4 * RunQuads<ACTK, LOWBIT_BITS>::n * 16)
int LOWBIT_CAT(qmv_stage_bytes_b, LOWBIT_BITS)(int act) {
  switch (act) {
    case ACT_F32: return LOWBIT_QMV_STAGE(ACT_F32);
    case ACT_F16: return LOWBIT_QMV_STAGE(ACT_F16);
    default: return LOWBIT_QMV_STAGE(ACT_BF16);
  }
}

}  // namespace lowbit
