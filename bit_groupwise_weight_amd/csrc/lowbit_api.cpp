// Host side of the C ABI declared in include/lowbit.h: argument validation,
// schedule selection and kernel dispatch.  Validation never touches the HIP
// runtime, so every argument error is reported identically with or without a
// GPU present.
#include "lowbit.h"
#include "lowbit_tuning.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <utility>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

lowbit_status fail(lowbit_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lowbit_status fail(lowbit_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

lowbit_status hip_fail(hipError_t e, const char* what) {
  return fail(LOWBIT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_bits(int bits) { return bits >= 1 && bits <= 7; }
bool valid_group(int g) { return g == 32 || g == 64 || g == 128 || g == 256; }
bool valid_dtype(lowbit_dtype d) { return d == LOWBIT_F32 || d == LOWBIT_F16 || d == LOWBIT_BF16; }
size_t dtype_bytes(lowbit_dtype d) { return d == LOWBIT_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shapes are limited so that every element index fits the kernels' 32-bit
// row/column counters and 64-bit offsets.
constexpr int64_t kMaxDim = int64_t(1) << 30;

lowbit_status check_common(int bits, int group, int64_t N, int64_t K) {
  if (!valid_bits(bits)) return fail(LOWBIT_ERR_INVALID_ARG, "bits=%d not in 1..7", bits);
  if (!valid_group(group))
    return fail(LOWBIT_ERR_INVALID_ARG, "group=%d not one of 32/64/128/256", group);
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim)
    return fail(LOWBIT_ERR_INVALID_ARG, "N=%lld K=%lld must be in 1..2^30", (long long)N,
                (long long)K);
  if (K % group != 0)
    return fail(LOWBIT_ERR_INVALID_ARG, "K=%lld is not a multiple of group=%d", (long long)K,
                group);
  return LOWBIT_OK;
}

// Arguments of one linear (shared by lowbit_linear_path and lowbit_linear_multi).
lowbit_status check_linear(const void* x, lowbit_dtype act_dtype, const uint8_t* packed,
                           const void* scales, const void* zeros, const void* bias, const void* y,
                           int bits, int group, int64_t M, int64_t N, int64_t K) {
  lowbit_status st = check_common(bits, group, N, K);
  if (st != LOWBIT_OK) return st;
  if (M < 0 || M > kMaxDim) return fail(LOWBIT_ERR_INVALID_ARG, "M=%lld", (long long)M);
  if (!valid_dtype(act_dtype)) return fail(LOWBIT_ERR_UNSUPPORTED, "act_dtype=%d", (int)act_dtype);
  if (!packed || !scales || !zeros) return fail(LOWBIT_ERR_INVALID_ARG, "NULL weight pointer");
  if (M > 0 && (!x || !y)) return fail(LOWBIT_ERR_INVALID_ARG, "NULL x or y");
  if (!aligned(packed, 16)) return fail(LOWBIT_ERR_MISALIGNED, "packed must be 16-byte aligned");
  if (!aligned(x, 16)) return fail(LOWBIT_ERR_MISALIGNED, "x must be 16-byte aligned");
  const size_t e = dtype_bytes(act_dtype);
  if (!aligned(scales, e) || !aligned(zeros, e) || !aligned(y, e) || (bias && !aligned(bias, e)))
    return fail(LOWBIT_ERR_MISALIGNED, "scales/zeros/bias/y must be aligned to their element size");
  return LOWBIT_OK;
}

// The quantizer's status words live in a device array that the library holds
// on every device (no allocation).  A call holds its device's mutex from
// clearing the words until it has read them back, so concurrent calls on one
// device (from any threads, on any streams) never see each other's flags.
constexpr int kMaxDevices = 64;
std::mutex g_status_mu[kMaxDevices];

// Current device's status words; on success *lock holds that device's mutex.
lowbit_status device_status_word(int** out, std::unique_lock<std::mutex>* lock) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LOWBIT_ERR_HIP, "device id %d out of range", dev);
  std::unique_lock<std::mutex> held(g_status_mu[dev]);
  e = lowbit::quant_status_words(out);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(status)");
  *lock = std::move(held);
  return LOWBIT_OK;
}

int act_kind(lowbit_dtype d) {
  switch (d) {
    case LOWBIT_F32: return lowbit::ACT_F32;
    case LOWBIT_F16: return lowbit::ACT_F16;
    default: return lowbit::ACT_BF16;
  }
}

typedef hipError_t (*QmvLauncher)(const lowbit::QmvBatch&, const lowbit::QmvLaunch&, int, int,
                                  hipStream_t);
const QmvLauncher kQmv[8] = {nullptr,
                             lowbit::launch_qmv_b1,
                             lowbit::launch_qmv_b2,
                             lowbit::launch_qmv_b3,
                             lowbit::launch_qmv_b4,
                             lowbit::launch_qmv_b5,
                             lowbit::launch_qmv_b6,
                             lowbit::launch_qmv_b7};

// Largest M that the automatic choice sends to the decode kernel: measured
// on MI355X at K = N = 4096, group 64, fp16 and bf16, b = 1..5 and 7 (both
// paths forced, graph-timed on one box) -- the decode kernel is faster up to
// M = 4 at every width (e.g. b = 4, fp16, M = 4: 7.7 vs 10.6 us) and the MFMA
// kernel from M = 5 (b = 4: 10.5 vs 11.2 us; b = 7: 12.7 vs 15.8 us): the
// decode kernel serves four activation rows per pass and re-reads the
// weights for the next four.
// Largest M the decode kernel takes by default: fp32 activations always go
// to it; fp16 from M = 3 and bf16 from M = 5 go to the MFMA kernels (the
// small-M kernel for fp16 up to 16 rows; measured at K = N = 4096, decode /
// small-M kernel, us: M = 2 5.1-6.8 / 5.4-7.6, M = 4 7.3-9.9 / 5.5-7.4,
// M = 8 10.8-16.4 / 6.6-8.2).
inline int64_t qmv_max_m(lowbit_dtype act) { return act == LOWBIT_F16 ? 2 : 4; }
static_assert(LOWBIT_MAX_MULTI <= lowbit::kQmvMaxProblems, "one launch serves every desc");

typedef int (*QmvStageBytes)(int);
const QmvStageBytes kQmvStage[8] = {nullptr,
                                    lowbit::qmv_stage_bytes_b1,
                                    lowbit::qmv_stage_bytes_b2,
                                    lowbit::qmv_stage_bytes_b3,
                                    lowbit::qmv_stage_bytes_b4,
                                    lowbit::qmv_stage_bytes_b5,
                                    lowbit::qmv_stage_bytes_b6,
                                    lowbit::qmv_stage_bytes_b7};

// LDS budget of one decode block for its staged activations.
constexpr int64_t kQmvStageBudget = 64 * 1024 - 256;

// Overrides of the automatic schedule choices (lowbit_set_tuning; 0 = none),
// for tests and benchmarks.  Nothing reads the environment.
std::atomic<int> g_tuning[LOWBIT_TUNE_COUNT] = {};

int tuning(lowbit_tuning_key key, int dflt) {
  const int v = g_tuning[key].load(std::memory_order_relaxed);
  return v != 0 ? v : dflt;
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// One decode problem of a (possibly multi-problem) launch.
struct QmvProblem {
  const void* x;
  const uint8_t* packed;
  const void* scales;
  const void* zeros;
  const void* bias;
  void* y;
  int64_t N, K;
};

// All problems share bits, group, activation dtype and M; one launch serves
// them all (blocks are dealt out to the problems in order).
lowbit_status run_qmv_multi(const QmvProblem* probs, int count, lowbit_dtype act, int bits, int group,
                            int64_t M, hipStream_t stream) {
  lowbit::QmvBatch b{};
  int max_shift = 0;
  int64_t max_per_row = 0;
  for (int i = 0; i < count; ++i) {
    const QmvProblem& q = probs[i];
    lowbit::QmvParams& p = b.prob[i];
    p.x = q.x; p.packed = q.packed; p.scales = q.scales; p.zeros = q.zeros; p.bias = q.bias; p.y = q.y;
    p.M = static_cast<int>(M);
    p.N = static_cast<int>(q.N);
    p.K = static_cast<int>(q.K);
    p.groups = static_cast<int>(q.K / group);
    p.row_bytes = q.K * bits / 8;
    // lanes per row group: enough for four 32-code runs each, at most 64
    const int64_t units = (q.K + 127) / 128;
    int shift = 0;
    while ((int64_t(1) << shift) < units && shift < 6) ++shift;
    p.lpr_shift = shift;
    max_shift = std::max(max_shift, shift);
    max_per_row = std::max<int64_t>(max_per_row,
                                    static_cast<int64_t>(kQmvStage[bits](act_kind(act))) << shift);
  }

  // Activation rows per pass: as many as fit the LDS stage (at most 4).
  // max_per_row holds 4 * quads-per-run * 16 bytes per lane, times the lanes.
  auto stage_bytes = [&](int mt) {
    const int64_t qd = (max_per_row >> max_shift) / (4 * 16);
    return static_cast<int64_t>(lowbit::qmv_stage_quads_per_lane(mt, static_cast<int>(qd))) * 16
           << max_shift;
  };
  lowbit::QmvLaunch l{};
  l.mt = 1;
  if (M >= 2 && stage_bytes(2) <= kQmvStageBudget) l.mt = 2;
  if (M >= 3 && stage_bytes(4) <= kQmvStageBudget) l.mt = 4;
  if (stage_bytes(1) > kQmvStageBudget) return fail(LOWBIT_ERR_UNSUPPORTED, "activation stage too large");
  // Block size: 256 threads unless that leaves fewer blocks than CUs.
  int threads = tuning(LOWBIT_TUNE_QMV_BLOCK, 0);
  auto blocks_for = [&](int t, int i, int variant) {
    const int64_t rows_per_block =
        static_cast<int64_t>(t >> b.prob[i].lpr_shift) * lowbit::qmv_rows_per_group(bits, l.mt, variant);
    return (probs[i].N + rows_per_block - 1) / rows_per_block;
  };
  auto total_blocks = [&](int t, int variant) {
    int64_t n = 0;
    for (int i = 0; i < count; ++i) n += blocks_for(t, i, variant);
    return n;
  };
  if (threads != 64 && threads != 128 && threads != 256) {
    threads = 256;
    while (threads > 64 && total_blocks(threads, lowbit::QMV_DEFAULT) < device_cus() &&
           (threads >> 1) >= (1 << max_shift))
      threads >>= 1;
  }
  if (threads < (1 << max_shift)) threads = 1 << max_shift;
  const int64_t by = (M + l.mt - 1) / l.mt;
  // One activation row: with more than two blocks per CU the lean variant
  // (one more wave per SIMD) gains 7-9 % at b = 4 from 4096 x 14336 to
  // 16384 x 16384 and 12 % at b = 1, 4096 x 14336 (3.5 blocks per CU), and
  // where two rows per lane group still leave six or more blocks per CU,
  // LEAN2 gains another ~10 % (4096 x 28672, 16384 x 16384; at 3.5-4 blocks
  // per CU it loses 0-3 %).  With two blocks per CU or fewer the default is
  // ahead by 0-3 % (K = N = 4096).
  // Rows of more than one round per lane (K > 128 * lanes, e.g. K = 14336)
  // also take the lean variant: b = 1/4/7 at K = 14336, N = 4096 run 3/9/11 %
  // faster with it at two to four blocks per CU.
  const int64_t cus = device_cus();
  bool multi_round = false;
  for (int i = 0; i < count; ++i)
    multi_round |= probs[i].K > (int64_t{128} << b.prob[i].lpr_shift);
  // Otherwise (one round, at most two blocks per CU), widths with two rows
  // per lane group take one row per lane group, which doubles the waves,
  // unless that leaves the CUs between two and four waves each.  A/B on one
  // box, us: K = 4096, N = 1024, b = 1, 2, 3: 3.81/3.96/4.09 -> 3.59/3.67/3.77
  // and K = 2048, N = 1024, b = 1, 3: 3.12/3.47 -> 2.71/3.10 (one wave per CU
  // before); K = N = 4096, b = 1, 3: 3.74/4.31 -> 3.67/4.22 and K = 4096,
  // N = 8192, b = 2, 3: 5.07/5.77 -> 4.92/5.37 (four and eight waves per CU
  // before); K = 4096, N = 2048 (two waves per CU before) loses 3 %.
  l.variant = lowbit::QMV_DEFAULT;
  const int64_t waves = total_blocks(threads, lowbit::QMV_DEFAULT) * by * (threads / 64);
  if (l.mt == 1 && (total_blocks(threads, lowbit::QMV_DEFAULT) * by > 2 * cus || multi_round))
    l.variant = total_blocks(threads, lowbit::QMV_LEAN2) * by >= 6 * cus ? lowbit::QMV_LEAN2 : lowbit::QMV_LEAN;
  else if (l.mt == 1 && (waves < 2 * cus || waves >= 4 * cus) &&
           lowbit::qmv_rows_per_group(bits, 1, lowbit::QMV_DEFAULT) == 2)
    l.variant = lowbit::QMV_LEAN1;
  const int var_env = tuning(LOWBIT_TUNE_QMV_VARIANT, 0) - 1;   // (override: 1..4 forces variant 0..3)
  if (l.mt == 1 && var_env >= 0 && var_env <= 3) l.variant = var_env;
  int64_t bx = 0;
  for (int i = 0; i < count; ++i) bx = std::max<int64_t>(bx, blocks_for(threads, i, l.variant));
  if (bx > 0x7fffffff || by > 65535) return fail(LOWBIT_ERR_INVALID_ARG, "problem too large");
  l.grid = dim3(static_cast<unsigned>(bx), static_cast<unsigned>(by), static_cast<unsigned>(count));
  l.block = dim3(threads);
  hipError_t e = kQmv[bits](b, l, group, act_kind(act), stream);
  if (e != hipSuccess) return hip_fail(e, "qmv launch");
  return LOWBIT_OK;
}

lowbit_status run_qmv(const void* x, lowbit_dtype act, const uint8_t* packed, const void* scales,
                      const void* zeros, const void* bias, void* y, int bits, int group,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const QmvProblem q{x, packed, scales, zeros, bias, y, N, K};
  return run_qmv_multi(&q, 1, act, bits, group, M, stream);
}

typedef hipError_t (*QmmLauncher)(const lowbit::QmmParams&, const lowbit::QmmLaunch&, int,
                                  hipStream_t);
const QmmLauncher kQmm[8] = {nullptr,
                             lowbit::launch_qmm_b1,
                             lowbit::launch_qmm_b2,
                             lowbit::launch_qmm_b3,
                             lowbit::launch_qmm_b4,
                             lowbit::launch_qmm_b5,
                             lowbit::launch_qmm_b6,
                             lowbit::launch_qmm_b7};

typedef hipError_t (*QmmSmallLauncher)(const lowbit::QmmParams&, int, int, hipStream_t);
const QmmSmallLauncher kQmmSmall[8] = {nullptr,
                                       lowbit::launch_qmm_small_b1,
                                       lowbit::launch_qmm_small_b2,
                                       lowbit::launch_qmm_small_b3,
                                       lowbit::launch_qmm_small_b4,
                                       lowbit::launch_qmm_small_b5,
                                       lowbit::launch_qmm_small_b6,
                                       lowbit::launch_qmm_small_b7};

// Schedule of the MFMA kernel: block tile (16*mtt) x (16*nt*waves), K steps
// of 128, and a K split that fills the CUs with one block each.
struct QmmSchedule {
  bool small;             // the small-M kernel (fields below: nt, waves only)
  int mtt, nt, waves, kgroups, rgroups;
  int64_t tiles_n, tiles_m, ksteps;
  int splits, ksteps_per_split;
  size_t partial_bytes;   // fp32 partial planes (split-K)
};

// Block tiles and K split for column tile width 16*nt*waves: one block per
// CU (each block takes a whole CU's register file), K split just enough that
// the tiles times the splits fill the CUs without a second, partial wave of
// blocks (LOWBIT_TUNE_QMM_BLOCKS overrides the block target).
void qmm_split(QmmSchedule& sc, int64_t M, int64_t N, int64_t K) {
  const int64_t bn = 16 * sc.nt * sc.waves;
  sc.tiles_n = (N + bn - 1) / bn;
  sc.tiles_m = (M + 16 * sc.mtt - 1) / (16 * sc.mtt);
  sc.ksteps = (K + 127) / 128;
  const int64_t target = tuning(LOWBIT_TUNE_QMM_BLOCKS, device_cus());
  const int64_t tiles = sc.tiles_n * sc.tiles_m;
  int64_t s = std::max<int64_t>(1, target / tiles);
  const int64_t max_split = std::max<int64_t>(1, sc.ksteps / 2);   // >= 2 steps per split
  s = std::max<int64_t>(1, std::min<int64_t>(s, std::min<int64_t>(max_split, 64)));
  sc.ksteps_per_split = static_cast<int>((sc.ksteps + s - 1) / s);
  // with two K groups, an even step count per split keeps the groups equal
  if (sc.kgroups == 2 && sc.ksteps_per_split % 2 == 1 && sc.ksteps_per_split < sc.ksteps)
    ++sc.ksteps_per_split;
  sc.splits = static_cast<int>((sc.ksteps + sc.ksteps_per_split - 1) / sc.ksteps_per_split);
  // partial planes cover whole block tiles (the reduce kernel skips the
  // records past M or N)
  sc.partial_bytes = 0;
  if (sc.splits > 1)
    sc.partial_bytes = static_cast<size_t>(sc.splits) * static_cast<size_t>(sc.tiles_n * bn) *
                       static_cast<size_t>(sc.tiles_m * 16 * sc.mtt) * sizeof(float);
}

// Steps per block at or below which 64-column blocks (one column tile per
// wave) beat 128-column ones at M = 128: the narrower tile halves the K split
// (no reduce kernel at all for N = 14336 with K <= 4096) at the price of
// twice the LDS reads per MFMA, which only pays while the loop is short
// (measured, N = 14336: K = 1024 13.1 vs 21.2 us, K = 2048 20.1 vs 24.7,
// K = 4096 even, K = 8192 62.7 vs 55.7; N = 4096: K = 7168 22.7 vs 24.4,
// K = 14336 36.0 vs 33.3).
constexpr int kQmmNarrowMaxSteps = 16;

// Two K groups need enough steps per block for their two-step pipeline:
// measured (A/B in alternating processes on one box) K groups win with 14-16
// steps per block (M = 128, K = 14336, N = 4096: 34.2 vs 35.0 us; M = 64,
// K = 4096, N = 14336: 30.8 vs 33.1; M = 32: 27.1 vs 28.4) and lose with 4
// (M = 64, K = N = 4096: 17.25 vs 16.8).
constexpr int kQmmKGroupsMinSteps = 8;

// Largest M of the small-M kernel (fp16 activations): it streams the weights
// once per call whatever M is, while the tiled kernel pays a K split, its
// reduce and a pipeline fill.
constexpr int kQmmSmallMaxM = 16;

QmmSchedule qmm_schedule(int bits, lowbit_dtype act, int64_t M, int64_t N, int64_t K) {
  QmmSchedule sc{};
  sc.rgroups = 1;
  const int small_env = tuning(LOWBIT_TUNE_QMM_SMALL_M, kQmmSmallMaxM);
  if (act == LOWBIT_F16 && M <= std::min(small_env, 16)) {
    // blocks of 16 columns (32 when asked) over all of K; waves per block so
    // that each takes at least two K steps
    const int64_t ksteps = (K + 127) / 128;
    sc.small = true;
    sc.nt = tuning(LOWBIT_TUNE_QMM_NT, 1) == 2 ? 2 : 1;
    sc.waves = ksteps >= 32 ? 16 : ksteps >= 16 ? 8 : 4;
    const int wv_env = tuning(LOWBIT_TUNE_QMM_WAVES, 0);
    if (wv_env == 4 || wv_env == 8 || wv_env == 16) sc.waves = wv_env;
    if (sc.nt == 2 && sc.waves == 16) sc.waves = 8;
    sc.mtt = 1;
    sc.kgroups = 1;
    sc.tiles_n = (N + 16 * sc.nt - 1) / (16 * sc.nt);
    sc.tiles_m = 1;
    sc.ksteps = ksteps;
    sc.splits = 1;
    sc.ksteps_per_split = static_cast<int>(ksteps);
    sc.partial_bytes = 0;
    return sc;
  }
  sc.mtt = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
  const int mtt_env = tuning(LOWBIT_TUNE_QMM_MTT, 0);
  if (mtt_env == 1 || mtt_env == 2 || mtt_env == 4 || mtt_env == 8) sc.mtt = std::min(sc.mtt, mtt_env);
  sc.nt = 2;
  if (act == LOWBIT_BF16) {
    // bf16: the code-operand kernel, 4 column waves of two column tiles;
    // 128-row tiles split between two row groups of 4 waves (two waves per
    // SIMD; 64-row tiles only when asked)
    sc.waves = 4;
    sc.kgroups = 1;
    const int rg_env = tuning(LOWBIT_TUNE_QMM_RGROUPS, 0);
    sc.rgroups = ((sc.mtt == 8 && rg_env != 1) || (sc.mtt == 4 && rg_env == 2)) ? 2 : 1;
    if (tuning(LOWBIT_TUNE_QMM_NT, 0) == 1) {
      sc.nt = 1;
      sc.rgroups = 1;
    }
    qmm_split(sc, M, N, K);
    return sc;
  }
  // Two K groups of 4 column waves (8 waves, 128 columns) keep two waves per
  // SIMD at the tile width of a 4-wave block, so the K split across blocks
  // stays that of the 4-wave block: one wave's dequantization runs under the
  // other's MFMAs.  Up to 4 bits, with at least kQmmKGroupsMinSteps steps per
  // block; 128-row tiles may narrow to one column tile per wave (below).
  // Otherwise one K group: 8 column waves (256 columns) for full 128-row
  // tiles when N is wide enough that the K split stays small (1.6x more work
  // per CU than 4-wave blocks at M = 128, K = 4096, N = 14336; the wider tile
  // needs twice the K splits, whose partial planes cost more than that gain
  // once the split exceeds ~4), else 4 waves.
  // (LOWBIT_TUNE_QMM_MTT, _KGROUPS, _WAVES and _NT override the choices;
  // _WAVES applies with one K group, _NT with two at 128-row tiles.)
  const bool can8 = bits <= lowbit::qmm_max_bits_8waves;
  const bool can_kg = bits <= lowbit::qmm_max_bits_kgroups;
  const int kg_env = tuning(LOWBIT_TUNE_QMM_KGROUPS, 0);
  if (can_kg && kg_env != 1) {
    QmmSchedule kg = sc;
    kg.kgroups = 2;
    kg.waves = 4;
    if (kg.mtt == 8) {
      QmmSchedule narrow = kg;
      narrow.nt = 1;
      qmm_split(narrow, M, N, K);
      const int nt_env = tuning(LOWBIT_TUNE_QMM_NT, 0);
      if (nt_env == 1 || (nt_env != 2 && narrow.ksteps_per_split <= kQmmNarrowMaxSteps)) return narrow;
    }
    qmm_split(kg, M, N, K);
    if (kg_env == 2 || kg.ksteps_per_split >= kQmmKGroupsMinSteps) return kg;
  }
  sc.kgroups = 1;
  const int wv_default = (can8 && sc.mtt == 8 && (N + 255) / 256 >= device_cus() / 5) ? 8 : 4;
  sc.waves = (can8 && tuning(LOWBIT_TUNE_QMM_WAVES, wv_default) == 8) ? 8 : 4;
  qmm_split(sc, M, N, K);
  return sc;
}

lowbit_status run_qmm(const void* x, lowbit_dtype act, const uint8_t* packed, const void* scales,
                      const void* zeros, const void* bias, void* y, int bits, int group,
                      int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  QmmSchedule sc = qmm_schedule(bits, act, M, N, K);
  if (sc.splits > 1 && (workspace == nullptr || workspace_bytes < sc.partial_bytes)) {
    sc.splits = 1;                               // no workspace: one block per tile over all K
    sc.ksteps_per_split = static_cast<int>(sc.ksteps);
  }
  if (sc.tiles_m > 65535 || sc.tiles_n > 0x7fffffff)
    return fail(LOWBIT_ERR_INVALID_ARG, "problem too large for qmm");
  // the bf16 kernel addresses activations and packed codes with 32-bit
  // lane offsets from a per-step base
  if (act == LOWBIT_BF16 && (M * K * 2 > int64_t{0xffffffff} || N * (K * bits / 8) > int64_t{0xffffffff}))
    return fail(LOWBIT_ERR_UNSUPPORTED, "bf16 qmm: activations and packed codes must each be below 4 GiB");
  if (sc.small) {
    lowbit::QmmParams p{};
    p.x = x; p.packed = packed; p.scales = scales; p.zeros = zeros; p.bias = bias; p.y = y;
    p.M = static_cast<int>(M);
    p.N = static_cast<int>(N);
    p.K = static_cast<int>(K);
    p.groups = static_cast<int>(K / group);
    int gs = 0;
    while ((1 << gs) < group) ++gs;
    p.group_shift = gs;
    p.row_bytes = K * bits / 8;
    p.ksteps_per_split = static_cast<int>(sc.ksteps);
    const hipError_t e = kQmmSmall[bits](p, sc.nt, sc.waves, stream);
    if (e != hipSuccess) return hip_fail(e, "small-M qmm launch");
    return LOWBIT_OK;
  }
  lowbit::QmmParams p{};
  p.x = x; p.packed = packed; p.scales = scales; p.zeros = zeros; p.bias = bias; p.y = y;
  p.M = static_cast<int>(M);
  p.N = static_cast<int>(N);
  p.K = static_cast<int>(K);
  p.groups = static_cast<int>(K / group);
  int gs = 0;
  while ((1 << gs) < group) ++gs;
  p.group_shift = gs;
  p.row_bytes = K * bits / 8;
  p.ksteps_per_split = sc.ksteps_per_split;
  if (sc.splits > 1) p.partials = static_cast<float*>(workspace);
  lowbit::QmmLaunch l{};
  l.mtt = sc.mtt;
  l.nt = sc.nt;
  l.waves = sc.waves;
  l.kgroups = sc.kgroups;
  l.rgroups = sc.rgroups;
  l.grid = dim3(static_cast<unsigned>(sc.tiles_n), static_cast<unsigned>(sc.tiles_m),
                static_cast<unsigned>(sc.splits));
  hipError_t e = kQmm[bits](p, l, act_kind(act), stream);
  if (e != hipSuccess) return hip_fail(e, "qmm launch");
  return LOWBIT_OK;
}

typedef hipError_t (*A8Launcher)(const lowbit::A8Params&, int, int, int, hipStream_t);
const A8Launcher kA8[8] = {nullptr,
                           lowbit::launch_qmm_a8_b1,
                           lowbit::launch_qmm_a8_b2,
                           lowbit::launch_qmm_a8_b3,
                           lowbit::launch_qmm_a8_b4,
                           lowbit::launch_qmm_a8_b5,
                           lowbit::launch_qmm_a8_b6,
                           lowbit::launch_qmm_a8_b7};

// Largest M of the int8-activation linear: 65535 blocks (the grid's y
// limit) of 16 rows.
constexpr int64_t kA8MaxM = int64_t(16) * 65535;

// Tiles of the int8-activation linear: 16-row tiles per block (mtt) and
// 16-column tiles per wave (nt).  The kernel is bound by its vector-memory
// instructions.  The block's waves share the activation fragments through
// LDS, so per 16 x 16 output tile and 64-wide K window a wave issues about
// 1/(4 nt) activation loads, 1/mtt code loads and 1/4 scale/zero loads: the
// row tiles matter most, and the largest tiles win as long as the launch
// keeps at least 3.5 waves per CU (measured at M = 128, bits 4, group 32:
// K = 4096, N = 14336 runs fastest with mtt 4, nt 1 at 7 waves per CU,
// 58 us, against 67 us for mtt 4, nt 2 at 3.5; K = 14336, N = 4096 with
// mtt 2, nt 1 at 4 waves per CU, 82 us, against 134-222 us for larger tiles
// at 2 waves per CU).
constexpr int kA8HalfWavesPerCu = 7;
void a8_tiles(int64_t M, int64_t N, int* mtt_out, int* nt_out) {
  static const int kOrder[][2] = {{4, 1}, {2, 1}, {4, 2}, {2, 2}, {1, 1}, {1, 2}};
  const int64_t target = (int64_t(kA8HalfWavesPerCu) * device_cus() + 1) / 2;
  int mtt = 1, nt = 1;
  for (const auto& c : kOrder) {
    if (c[0] > 1 && 16 * (c[0] / 2) >= M) continue;   // the rows fit in half the tiles
    const int64_t waves = ((N + 16 * c[1] - 1) / (16 * c[1])) * ((M + 16 * c[0] - 1) / (16 * c[0]));
    if (waves >= target) {
      mtt = c[0];
      nt = c[1];
      break;
    }
  }
  const int fm = tuning(LOWBIT_TUNE_A8_MTT, 0), fn = tuning(LOWBIT_TUNE_A8_NT, 0);
  if (fm == 1 || fm == 2 || fm == 4) mtt = fm;
  if (fn == 1 || fn == 2) nt = fn;
  *mtt_out = mtt;
  *nt_out = nt;
}

}  // namespace

extern "C" {

int lowbit_abi_version(void) { return LOWBIT_ABI_VERSION; }

size_t lowbit_packed_bytes(int bits, int64_t N, int64_t K) {
  if (!valid_bits(bits) || N <= 0 || K <= 0 || K % 32 != 0) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) * bits / 8;
}

int64_t lowbit_num_groups(int64_t K, int group) {
  if (!valid_group(group) || K <= 0 || K % group != 0) return 0;
  return K / group;
}

const char* lowbit_status_string(lowbit_status s) {
  switch (s) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_ERR_INVALID_ARG: return "invalid argument";
    case LOWBIT_ERR_UNSUPPORTED: return "unsupported combination";
    case LOWBIT_ERR_MISALIGNED: return "misaligned pointer";
    case LOWBIT_ERR_NONFINITE: return "non-finite weight";
    case LOWBIT_ERR_RANGE: return "scale or zero out of range for its dtype";
    case LOWBIT_ERR_WORKSPACE: return "bad workspace";
    case LOWBIT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* lowbit_last_error(void) { return g_last_error.c_str(); }

lowbit_status lowbit_set_tuning(lowbit_tuning_key key, int value) {
  g_last_error.clear();
  if (static_cast<int>(key) < 0 || key >= LOWBIT_TUNE_COUNT)
    return fail(LOWBIT_ERR_INVALID_ARG, "tuning key %d", (int)key);
  if (value < 0) return fail(LOWBIT_ERR_INVALID_ARG, "tuning value %d", value);
  g_tuning[key].store(value, std::memory_order_relaxed);
  return LOWBIT_OK;
}

lowbit_status lowbit_quantize_pack(const void* w, lowbit_dtype w_dtype, int bits, int group, int64_t N,
                                   int64_t K, lowbit_dtype sz_dtype, void* scales, void* zeros,
                                   uint8_t* packed, uint8_t* codes, void* stream) {
  g_last_error.clear();
  lowbit_status st = check_common(bits, group, N, K);
  if (st != LOWBIT_OK) return st;
  if (!valid_dtype(w_dtype)) return fail(LOWBIT_ERR_UNSUPPORTED, "w_dtype=%d", (int)w_dtype);
  if (!valid_dtype(sz_dtype)) return fail(LOWBIT_ERR_UNSUPPORTED, "sz_dtype=%d", (int)sz_dtype);
  if (!w || !scales || !zeros || !packed) return fail(LOWBIT_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(w, 16)) return fail(LOWBIT_ERR_MISALIGNED, "w must be 16-byte aligned");
  if (!aligned(packed, 16)) return fail(LOWBIT_ERR_MISALIGNED, "packed must be 16-byte aligned");
  const size_t e = dtype_bytes(sz_dtype);
  if (!aligned(scales, e) || !aligned(zeros, e))
    return fail(LOWBIT_ERR_MISALIGNED, "scales/zeros must be aligned to their element size");

  hipStream_t s = static_cast<hipStream_t>(stream);
  int* status = nullptr;
  std::unique_lock<std::mutex> status_lock;
  st = device_status_word(&status, &status_lock);
  if (st != LOWBIT_OK) return st;
  hipError_t he = hipMemsetAsync(status, 0, 2 * sizeof(int), s);
  if (he != hipSuccess) return hip_fail(he, "hipMemsetAsync(status)");
  lowbit::QuantParams p{};
  p.w = w; p.scales = scales; p.zeros = zeros; p.packed = packed; p.codes = codes;
  p.status = status; p.N = N; p.K = K; p.bits = bits; p.group = group;
  p.sz_act = act_kind(sz_dtype);
  p.w_act = act_kind(w_dtype);
  he = lowbit::launch_quant_pack(p, s);
  if (he != hipSuccess) return hip_fail(he, "quant_pack launch");
  int host[2] = {0, 0};
  he = hipMemcpyAsync(host, status, sizeof(host), hipMemcpyDeviceToHost, s);
  if (he != hipSuccess) return hip_fail(he, "hipMemcpyAsync(status)");
  he = hipStreamSynchronize(s);
  if (he != hipSuccess) return hip_fail(he, "hipStreamSynchronize");
  if (host[0]) return fail(LOWBIT_ERR_NONFINITE, "weight holds a NaN or infinity");
  if (host[1]) return fail(LOWBIT_ERR_RANGE, "a scale or zero is not finite in its dtype");
  return LOWBIT_OK;
}

size_t lowbit_linear_workspace_bytes(int bits, int group, int64_t M, int64_t N, int64_t K,
                                     lowbit_dtype act_dtype) {
  if (!valid_bits(bits) || !valid_group(group) || M <= 0 || N <= 0 || K <= 0 || K % group != 0 ||
      M > kMaxDim || N > kMaxDim || K > kMaxDim || !valid_dtype(act_dtype))
    return 0;
  if (act_dtype == LOWBIT_F32) return 0;         // fp32 runs the decode kernel only
  const QmmSchedule sc = qmm_schedule(bits, act_dtype, M, N, K);
  return sc.partial_bytes;
}

lowbit_status lowbit_linear_path(const void* x, lowbit_dtype act_dtype, const uint8_t* packed,
                                 const void* scales, const void* zeros, const void* bias, void* y,
                                 int bits, int group, int64_t M, int64_t N, int64_t K,
                                 void* workspace, size_t workspace_bytes, lowbit_path path,
                                 void* stream) {
  g_last_error.clear();
  lowbit_status st = check_linear(x, act_dtype, packed, scales, zeros, bias, y, bits, group, M, N, K);
  if (st != LOWBIT_OK) return st;
  if (path != LOWBIT_PATH_AUTO && path != LOWBIT_PATH_QMV && path != LOWBIT_PATH_QMM)
    return fail(LOWBIT_ERR_INVALID_ARG, "path=%d", (int)path);
  if (workspace == nullptr && workspace_bytes != 0)
    return fail(LOWBIT_ERR_WORKSPACE, "workspace_bytes > 0 with a NULL workspace");
  if (workspace != nullptr && !aligned(workspace, 256))
    return fail(LOWBIT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (path == LOWBIT_PATH_QMM && act_dtype == LOWBIT_F32)
    return fail(LOWBIT_ERR_UNSUPPORTED, "the MFMA path takes fp16 or bf16 activations");
  if (M == 0) return LOWBIT_OK;

  bool use_qmm;
  if (path == LOWBIT_PATH_QMV) use_qmm = false;
  else if (path == LOWBIT_PATH_QMM) use_qmm = true;
  else use_qmm = (M > qmv_max_m(act_dtype)) && act_dtype != LOWBIT_F32;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_qmm)
    return run_qmm(x, act_dtype, packed, scales, zeros, bias, y, bits, group, M, N, K, workspace,
                   workspace_bytes, s);
  return run_qmv(x, act_dtype, packed, scales, zeros, bias, y, bits, group, M, N, K, s);
}

lowbit_status lowbit_linear(const void* x, lowbit_dtype act_dtype, const uint8_t* packed,
                            const void* scales, const void* zeros, const void* bias, void* y,
                            int bits, int group, int64_t M, int64_t N, int64_t K, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return lowbit_linear_path(x, act_dtype, packed, scales, zeros, bias, y, bits, group, M, N, K,
                            workspace, workspace_bytes, LOWBIT_PATH_AUTO, stream);
}

lowbit_status lowbit_linear_noalloc(const void* x, lowbit_dtype act_dtype, const uint8_t* packed,
                                    const void* scales, const void* zeros, const void* bias, void* y,
                                    int bits, int group, int64_t M, int64_t N, int64_t K,
                                    void* stream) {
  g_last_error.clear();
  lowbit_status st = check_linear(x, act_dtype, packed, scales, zeros, bias, y, bits, group, M, N, K);
  if (st != LOWBIT_OK) return st;
  if (M == 0) return LOWBIT_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool use_qmm = (M > qmv_max_m(act_dtype)) && act_dtype != LOWBIT_F32;
  if (!use_qmm) return run_qmv(x, act_dtype, packed, scales, zeros, bias, y, bits, group, M, N, K, s);
  // the schedule lowbit_linear takes with a full workspace, its partial
  // planes in the library's device array
  const QmmSchedule sc = qmm_schedule(bits, act_dtype, M, N, K);
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (sc.partial_bytes > 0) {
    if (sc.partial_bytes > lowbit::kNoallocScratchBytes)
      return fail(LOWBIT_ERR_WORKSPACE,
                  "this problem's K split needs %zu bytes of scratch, more than the %zu bytes of the "
                  "library's device array; call lowbit_linear with a workspace",
                  sc.partial_bytes, lowbit::kNoallocScratchBytes);
    const hipError_t e = lowbit::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    scratch_bytes = lowbit::kNoallocScratchBytes;
  }
  return run_qmm(x, act_dtype, packed, scales, zeros, bias, y, bits, group, M, N, K, scratch,
                 scratch_bytes, s);
}

lowbit_status lowbit_linear_multi(const lowbit_linear_desc* descs, int count, lowbit_dtype act_dtype,
                                  int bits, int group, int64_t M, void* stream) {
  g_last_error.clear();
  if (count < 0 || count > LOWBIT_MAX_MULTI)
    return fail(LOWBIT_ERR_INVALID_ARG, "count=%d not in 0..%d", count, LOWBIT_MAX_MULTI);
  if (count > 0 && descs == nullptr) return fail(LOWBIT_ERR_INVALID_ARG, "NULL descs");
  QmvProblem probs[LOWBIT_MAX_MULTI];
  for (int i = 0; i < count; ++i) {
    const lowbit_linear_desc& d = descs[i];
    const lowbit_status st = check_linear(d.x, act_dtype, d.packed, d.scales, d.zeros, d.bias, d.y,
                                          bits, group, M, d.N, d.K);
    if (st != LOWBIT_OK) {
      const std::string detail = g_last_error;
      return fail(st, "desc %d: %s", i, detail.c_str());
    }
    probs[i] = QmvProblem{d.x, d.packed, d.scales, d.zeros, d.bias, d.y, d.N, d.K};
  }
  if (count == 0 || M == 0) return LOWBIT_OK;
  return run_qmv_multi(probs, count, act_dtype, bits, group, M, static_cast<hipStream_t>(stream));
}

lowbit_status lowbit_quantize_act_i8(const void* x, lowbit_dtype act_dtype, int64_t M, int64_t K,
                                     int8_t* xq, float* ascale, void* stream) {
  g_last_error.clear();
  if (!valid_dtype(act_dtype)) return fail(LOWBIT_ERR_UNSUPPORTED, "act_dtype=%d", (int)act_dtype);
  if (M < 0 || M > kMaxDim) return fail(LOWBIT_ERR_INVALID_ARG, "M=%lld", (long long)M);
  if (K <= 0 || K > kMaxDim || K % 32 != 0)
    return fail(LOWBIT_ERR_INVALID_ARG, "K=%lld must be a positive multiple of 32 (at most 2^30)",
                (long long)K);
  if (M == 0) return LOWBIT_OK;
  if (!x || !xq || !ascale) return fail(LOWBIT_ERR_INVALID_ARG, "NULL x, xq or ascale");
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(ascale, 4))
    return fail(LOWBIT_ERR_MISALIGNED, "x and xq must be 16-byte aligned, ascale 4-byte aligned");
  lowbit::ActQuantParams p{x, xq, ascale, static_cast<int>(M), static_cast<int>(K)};
  const hipError_t e = lowbit::launch_act_quant_i8(p, act_kind(act_dtype), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "act_quant_i8 launch");
  return LOWBIT_OK;
}

lowbit_status lowbit_linear_a8(const int8_t* xq, const float* ascale, const uint8_t* packed,
                               const void* scales, const void* zeros, const void* bias, void* y,
                               lowbit_dtype dtype, int bits, int group, int64_t M, int64_t N,
                               int64_t K, void* stream) {
  g_last_error.clear();
  lowbit_status st = check_common(bits, group, N, K);
  if (st != LOWBIT_OK) return st;
  if (M < 0 || M > kA8MaxM)
    return fail(LOWBIT_ERR_INVALID_ARG, "M=%lld not in 0..%lld", (long long)M, (long long)kA8MaxM);
  if (!valid_dtype(dtype)) return fail(LOWBIT_ERR_UNSUPPORTED, "dtype=%d", (int)dtype);
  if (!packed || !scales || !zeros) return fail(LOWBIT_ERR_INVALID_ARG, "NULL weight pointer");
  if (M == 0) return LOWBIT_OK;
  if (!xq || !ascale || !y) return fail(LOWBIT_ERR_INVALID_ARG, "NULL xq, ascale or y");
  if (!aligned(packed, 16) || !aligned(xq, 16))
    return fail(LOWBIT_ERR_MISALIGNED, "packed and xq must be 16-byte aligned");
  const size_t e = dtype_bytes(dtype);
  if (!aligned(ascale, 4) || !aligned(scales, e) || !aligned(zeros, e) || !aligned(y, e) ||
      (bias && !aligned(bias, e)))
    return fail(LOWBIT_ERR_MISALIGNED, "ascale/scales/zeros/bias/y must be aligned to their element size");
  lowbit::A8Params p{};
  p.xq = xq;
  p.ascale = ascale;
  p.packed = packed;
  p.scales = scales;
  p.zeros = zeros;
  p.bias = bias;
  p.y = y;
  p.M = static_cast<int>(M);
  p.N = static_cast<int>(N);
  p.K = static_cast<int>(K);
  p.groups = static_cast<int>(K / group);
  p.group = group;
  p.row_bytes = K * bits / 8;
  int mtt = 1, nt = 1;
  a8_tiles(M, N, &mtt, &nt);
  const hipError_t he = kA8[bits](p, mtt, nt, act_kind(dtype), static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "qmm_a8 launch");
  return LOWBIT_OK;
}

}  // extern "C"