// Launch interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

// Activation (and scale/zero) element types.
enum ActKind : int { ACT_F32 = 0, ACT_F16 = 1, ACT_BF16 = 2 };

// ---------------------------------------------------------------- quantize --
struct QuantParams {
  const void* w;       // N x K, w_act (fp32, fp16 or bf16; upcast exactly to fp32)
  void* scales;        // N x G, sz dtype
  void* zeros;         // N x G, sz dtype
  uint8_t* packed;     // N x K*bits/8
  uint8_t* codes;      // N x K or nullptr
  int* status;         // [0] non-finite weight seen, [1] non-finite stored scale/zero
  int64_t N, K;
  int bits, group, sz_act, w_act;
};
hipError_t launch_quant_pack(const QuantParams& p, hipStream_t stream);

// --------------------------------------------------------------------- qmv --
struct QmvParams {
  const void* x;          // M x K act
  const uint8_t* packed;  // N x row_bytes
  const void* scales;     // N x groups act
  const void* zeros;      // N x groups act
  const void* bias;       // N act or nullptr
  void* y;                // M x N act
  int M, N, K;
  int lpr_shift;          // log2(lanes cooperating on one row group), <= 6
  int groups;             // K / group
  int64_t row_bytes;      // K * bits / 8
};
// Variants of the decode kernel for one activation row per pass (chosen at
// launch from the blocks per CU, the waves per CU and the row length): the
// default; LEAN, which keeps one staged fragment live at a time (fewer
// registers, one more wave per SIMD); LEAN2, LEAN with two rows per lane
// group at every bit width (more weight bytes in flight per wave); and LEAN1,
// LEAN with one row per lane group at every bit width (twice the waves where
// the default has two rows, for launches too small to fill the CUs).
enum QmvVariant { QMV_DEFAULT = 0, QMV_LEAN = 1, QMV_LEAN2 = 2, QMV_LEAN1 = 3 };
// Rows per row group of the decode kernel for one activation row per pass:
// two rows for 1, 2 and 3-bit codes, one for 4..7 bits (measured on MI355X at
// K = N = 4096, A/B of both builds on one box: two rows 0.15-0.18 us faster
// at b = 1, 2, equal at b = 3, 4, 6, 7, one row 0.35 us faster at b = 5),
// two for every width in LEAN2, one in LEAN1; one row whenever several
// activation rows share a pass.
constexpr int qmv_rows_per_group(int bits, int mt, int variant) {
  return mt == 1 && variant != QMV_LEAN1 && (variant == QMV_LEAN2 || bits <= 3) ? 2 : 1;
}
// LDS quads (16 bytes) per lane of a row group that the decode kernel stages
// for `mt` activation rows of `qd` quads per run (four runs per lane): rounded
// up to an odd count, so that the 16 lanes of one 16-byte LDS read, each at
// the same quad of its own runs, start in 16 distinct 4-bank groups.
constexpr int qmv_stage_quads_per_lane(int mt, int qd) { return (mt * 4 * qd) | 1; }
// Up to kQmvMaxProblems decode problems of one bit width, group size and
// activation dtype served by one launch: blocks with blockIdx.z == i work on
// problem i (grid.x is sized for the largest; blocks past a problem's rows
// exit at once); all share M (grid.y).
constexpr int kQmvMaxProblems = 8;
struct QmvBatch {
  QmvParams prob[kQmvMaxProblems];
};
struct QmvLaunch {
  dim3 grid, block;
  int mt;                 // activation rows per pass: 1, 2 or 4
  int variant;            // mt == 1: a QmvVariant
};
// One entry point per bit width (compiled as separate objects).
hipError_t launch_qmv_b1(const QmvBatch&, const QmvLaunch&, int group, int act, hipStream_t);
hipError_t launch_qmv_b2(const QmvBatch&, const QmvLaunch&, int group, int act, hipStream_t);
hipError_t launch_qmv_b3(const QmvBatch&, const QmvLaunch&, int group, int act, hipStream_t);
hipError_t launch_qmv_b4(const QmvBatch&, const QmvLaunch&, int group, int act, hipStream_t);
hipError_t launch_qmv_b5(const QmvBatch&, const QmvLaunch&, int group, int act, hipStream_t);
hipError_t launch_qmv_b6(const QmvBatch&, const QmvLaunch&, int group, int act, hipStream_t);
hipError_t launch_qmv_b7(const QmvBatch&, const QmvLaunch&, int group, int act, hipStream_t);
// LDS bytes the decode kernel stages per activation row and per lane of a
// round (four 32-code runs).
int qmv_stage_bytes_b1(int act);
int qmv_stage_bytes_b2(int act);
int qmv_stage_bytes_b3(int act);
int qmv_stage_bytes_b4(int act);
int qmv_stage_bytes_b5(int act);
int qmv_stage_bytes_b6(int act);
int qmv_stage_bytes_b7(int act);

// --------------------------------------------------------------------- qmm --
struct QmmParams {
  const void* x;          // M x K act (f16 / bf16)
  const uint8_t* packed;  // N x row_bytes
  const void* scales;     // N x groups act
  const void* zeros;      // N x groups act
  const void* bias;       // N act or nullptr
  void* y;                // M x N act
  float* partials;        // split-K: gridDim.z planes of fp32 tile records (workspace)
  int M, N, K;
  int groups;             // K / group
  int group_shift;        // log2(group)
  int ksteps_per_split;   // 128-wide K steps per grid.z slice
  int64_t row_bytes;      // K * bits / 8
};
// Layout of the split-K partial planes for the reduce kernel: records of
// 4 fp32 in (tile, wave, row tile, column tile, lane) order, one plane per
// K split (block tile 16*mtt x 16*nt*waves; mtt, nt, waves powers of two).
struct QmmReduceShape {
  int splits;
  int tiles_n;            // gridDim.x of the main kernel
  int mtt_shift, nt_shift, wv_shift;
  int64_t plane_recs;     // records per plane
};
// Largest bit widths with an 8-wave MFMA kernel instance: 8 column waves,
// and 4 column waves in two K groups (whose super-step activations take more
// registers).
constexpr int qmm_max_bits_8waves = 5;
constexpr int qmm_max_bits_kgroups = 4;
struct QmmLaunch {
  dim3 grid;              // (ceil(N/(16*nt*waves)), ceil(M/(16*mtt)), k-splits)
  int mtt;                // 16-row MFMA tiles per block: 1, 2, 4 or 8
  int nt;                 // 16-column MFMA tiles per wave (2)
  int waves;              // column waves per block: 4, or 8 (bits <= qmm_max_bits_8waves)
  int kgroups;            // K groups per block: 1, or 2 with 4 column waves
                          // (bits <= qmm_max_bits_kgroups); waves*kgroups waves in all
  int rgroups;            // bf16 kernel: row groups per block, 1 or 2 (each a set of
                          // `waves` column waves over its share of the row tiles)
};
hipError_t launch_qmm_b1(const QmmParams&, const QmmLaunch&, int act, hipStream_t);
hipError_t launch_qmm_b2(const QmmParams&, const QmmLaunch&, int act, hipStream_t);
hipError_t launch_qmm_b3(const QmmParams&, const QmmLaunch&, int act, hipStream_t);
hipError_t launch_qmm_b4(const QmmParams&, const QmmLaunch&, int act, hipStream_t);
hipError_t launch_qmm_b5(const QmmParams&, const QmmLaunch&, int act, hipStream_t);
hipError_t launch_qmm_b6(const QmmParams&, const QmmLaunch&, int act, hipStream_t);
hipError_t launch_qmm_b7(const QmmParams&, const QmmLaunch&, int act, hipStream_t);
// The small-M MFMA kernel (1 <= M <= 16, fp16 activations): blocks of
// 16*nt columns (nt 1 or 2) over all of K, `waves` (4, 8 or 16) waves per
// block splitting the K steps; no workspace, one launch.
hipError_t launch_qmm_small_b1(const QmmParams&, int nt, int waves, hipStream_t);
hipError_t launch_qmm_small_b2(const QmmParams&, int nt, int waves, hipStream_t);
hipError_t launch_qmm_small_b3(const QmmParams&, int nt, int waves, hipStream_t);
hipError_t launch_qmm_small_b4(const QmmParams&, int nt, int waves, hipStream_t);
hipError_t launch_qmm_small_b5(const QmmParams&, int nt, int waves, hipStream_t);
hipError_t launch_qmm_small_b6(const QmmParams&, int nt, int waves, hipStream_t);
hipError_t launch_qmm_small_b7(const QmmParams&, int nt, int waves, hipStream_t);
// The bf16 kernel's main launch (code operands; 4 column waves, nt == 2,
// one K group); launch_qmm_b<bits> calls it and adds the split-K reduce.
hipError_t launch_qmm_bf16_b1(const QmmParams&, const QmmLaunch&, hipStream_t);
hipError_t launch_qmm_bf16_b2(const QmmParams&, const QmmLaunch&, hipStream_t);
hipError_t launch_qmm_bf16_b3(const QmmParams&, const QmmLaunch&, hipStream_t);
hipError_t launch_qmm_bf16_b4(const QmmParams&, const QmmLaunch&, hipStream_t);
hipError_t launch_qmm_bf16_b5(const QmmParams&, const QmmLaunch&, hipStream_t);
hipError_t launch_qmm_bf16_b6(const QmmParams&, const QmmLaunch&, hipStream_t);
hipError_t launch_qmm_bf16_b7(const QmmParams&, const QmmLaunch&, hipStream_t);

// ------------------------------------------- int8 dynamic activations --
struct ActQuantParams {
  const void* x;          // M x K act (fp32, fp16 or bf16), 16-byte aligned
  int8_t* xq;             // M x K codes, 16-byte aligned
  float* ascale;          // M
  int M, K;               // K % 16 == 0
};
hipError_t launch_act_quant_i8(const ActQuantParams&, int act, hipStream_t);

struct A8Params {
  const int8_t* xq;       // M x K codes, 16-byte aligned
  const float* ascale;    // M
  const uint8_t* packed;  // N x row_bytes
  const void* scales;     // N x groups, sz dtype
  const void* zeros;      // N x groups, sz dtype
  const void* bias;       // N, sz dtype, or nullptr
  void* y;                // M x N, sz dtype
  int M, N, K;
  int groups;             // K / group
  int group;
  int64_t row_bytes;      // K * bits / 8
};
// Blocks of 4 waves, `nt` (1 or 2) 16-column MFMA tiles per wave, `mtt`
// (1, 2 or 4) 16-row tiles per block: grid (ceil(N / (64 nt)), ceil(M / (16 mtt))).
hipError_t launch_qmm_a8_b1(const A8Params&, int mtt, int nt, int sz, hipStream_t);
hipError_t launch_qmm_a8_b2(const A8Params&, int mtt, int nt, int sz, hipStream_t);
hipError_t launch_qmm_a8_b3(const A8Params&, int mtt, int nt, int sz, hipStream_t);
hipError_t launch_qmm_a8_b4(const A8Params&, int mtt, int nt, int sz, hipStream_t);
hipError_t launch_qmm_a8_b5(const A8Params&, int mtt, int nt, int sz, hipStream_t);
hipError_t launch_qmm_a8_b6(const A8Params&, int mtt, int nt, int sz, hipStream_t);
hipError_t launch_qmm_a8_b7(const A8Params&, int mtt, int nt, int sz, hipStream_t);

// ------------------------------------------------- library-owned scratch --
// Size of the device array behind lowbit_linear_noalloc (per device).  The
// largest K-split schedule of the MFMA path writes one fp32 partial per
// output of a block tile per block, at most (CUs) x (128 x 256) x 4 bytes =
// 32 MiB on a 256-CU device.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
// Device address of this device's copy of the array (looked up once per
// device, with that device current).
hipError_t noalloc_scratch(void** out);
// Device address of this device's two status words of the quantizer (a
// second library-owned device array, looked up the same way).
hipError_t quant_status_words(int** out);

}  // namespace lowbit
