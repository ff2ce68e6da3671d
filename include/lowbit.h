/*
 * lowbit.h -- C ABI of the groupwise weight-only low-bit linear layer for
 * AMD MI355X (gfx950).
 *
 *   y[M, N] = x[M, K] . dequant(Wq)[N, K]^T (+ bias[N])
 *   dequant(Wq)[n, k] = s[n, k / group] * q[n, k] + z[n, k / group]
 *
 * The operation and its weight format come from these pages:
 *   - "Add torchao mps ops": the linear:afpwx scheme -- weights only, quantized
 *     groupwise with a bit width of 1..7 and a group size of 32, 64, 128 or 256;
 *     activations stay floating point.
 *   - "metal lowbit kernels: qmv_fast optimization", Summary: scales and zeros
 *     are consumed N x num_groups (as the quantize function produces them), and
 *     codes are stored contiguously, carrying over into the next byte when the
 *     current byte is full.  The same page's closing question -- whether the
 *     decode matrix-vector approach also serves a matrix-matrix product -- is
 *     answered here by a separate MFMA path for larger M.
 *   - "Revamp int4 MPS support in torchao": the layer must accept a bias.
 *   - "Add support for fbgemm int4 mm kernel": configuration is passed as
 *     integers and enums, not strings (the review comment on that page).
 *
 * Conventions fixed where the pages are silent:
 *   - dequantization is w = s*q + z; z is a real-valued offset stored in the
 *     same dtype as s (the activation dtype);
 *   - quantization is asymmetric min/max per (row, group):
 *       s = (max - min) / (2^b - 1), z = min (a zero min/max counts as +0),
 *       s and z are rounded to their storage dtype (nearest even) first, then
 *       q = clamp(rint_half_even((w - z) / s), 0, 2^b - 1) in fp32 with a
 *       correctly rounded divide, and q = 0 where the stored s is 0;
 *   - packing: row n occupies bytes [n*K*b/8, (n+1)*K*b/8) of `packed`; bit j
 *     of code q[n,k] is bit (p & 7) of byte (p >> 3) of that row, p = k*b + j
 *     (least significant bit first), no padding.
 *
 * Memory: every pointer argument other than `stream` and the host-side helpers
 * is a DEVICE pointer owned by the caller; the library never keeps a pointer
 * after a call returns.  The library allocates no device memory: it holds,
 * on every device it runs on, two small arrays of its own (the quantizer's
 * status words and the scratch of lowbit_linear_noalloc).  Measurement
 * probes live in a separate library (lowbit_probe.h); schedule overrides
 * for tests and benchmarks in lowbit_tuning.h.
 *
 * Errors: arguments are validated on the host before any HIP call, so every
 * LOWBIT_ERR_INVALID_ARG / UNSUPPORTED / MISALIGNED / WORKSPACE result can be
 * produced without a GPU.  A failed HIP call yields LOWBIT_ERR_HIP; the text of
 * the last error on the calling thread is available from lowbit_last_error().
 * No C++ exception crosses this interface.
 */
#ifndef LOWBIT_H_
#define LOWBIT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWBIT_ABI_VERSION 3

typedef enum lowbit_status {
  LOWBIT_OK = 0,
  LOWBIT_ERR_INVALID_ARG = 1,  /* bits/group/shape out of range, NULL pointer      */
  LOWBIT_ERR_UNSUPPORTED = 2,  /* a dtype or path combination that is not built     */
  LOWBIT_ERR_MISALIGNED = 3,   /* packed, x (linear) or w (quantize) not 16-byte
                                  aligned, or another array not aligned to its
                                  element size                                      */
  LOWBIT_ERR_NONFINITE = 4,    /* quantize: the weight holds a NaN or an infinity   */
  LOWBIT_ERR_RANGE = 5,        /* quantize: a scale or zero overflows its dtype     */
  LOWBIT_ERR_WORKSPACE = 6,    /* workspace pointer/size inconsistent               */
  LOWBIT_ERR_HIP = 7           /* a HIP runtime call or kernel launch failed        */
} lowbit_status;

typedef enum lowbit_dtype {
  LOWBIT_F32 = 0,
  LOWBIT_F16 = 1,
  LOWBIT_BF16 = 2
} lowbit_dtype;

/* Which kernel family lowbit_linear_path runs. */
typedef enum lowbit_path {
  LOWBIT_PATH_AUTO = 0,  /* qmv for fp32 activations, fp16 at M <= 2 and
                            bf16 at M <= 4; qmm otherwise */
  LOWBIT_PATH_QMV = 1,   /* decode matrix-vector kernel, any M              */
  LOWBIT_PATH_QMM = 2    /* MFMA kernels, fp16/bf16 only (fp16 at M <= 16:
                            the small-M kernel, no workspace)               */
} lowbit_path;

/* ABI version of the loaded library (LOWBIT_ABI_VERSION at build time). */
int lowbit_abi_version(void);

/* Bytes of one packed weight matrix: N*K*bits/8.  Returns 0 when bits is not
 * in 1..7, N or K is not positive, or K is not a multiple of 32. */
size_t lowbit_packed_bytes(int bits, int64_t N, int64_t K);

/* K / group, or 0 when group is not 32/64/128/256 or K is not a positive
 * multiple of group. */
int64_t lowbit_num_groups(int64_t K, int group);

/* Quantize and pack a weight matrix (one-off, not on the decode path).
 *
 *   w        device, N x K row-major (the linear weight, [out, in]), 16-byte
 *            aligned.
 *   w_dtype  dtype of w: fp32, or fp16 / bf16, whose values are taken exactly
 *            as fp32 (every fp16 and bf16 value is an fp32 value).
 *   bits     1..7;  group: 32, 64, 128 or 256;  K % group == 0;  N, K > 0.
 *   sz_dtype storage dtype of scales and zeros; use the activation dtype that
 *            lowbit_linear will be called with.
 *   scales   device, N x (K/group) row-major, sz_dtype.  Written.
 *   zeros    device, N x (K/group) row-major, sz_dtype.  Written.
 *   packed   device, lowbit_packed_bytes(bits, N, K) bytes, 16-byte aligned.
 *            Written (every byte).
 *   codes    device, N x K bytes holding one code per byte, or NULL.
 *   stream   hipStream_t (NULL = the default stream).
 *
 * The call enqueues the work on `stream` and then waits for that stream,
 * because it reports data-dependent errors: LOWBIT_ERR_NONFINITE if w holds a
 * NaN or infinity, LOWBIT_ERR_RANGE if a scale or zero is not finite in
 * sz_dtype.  On either error the output buffers hold unspecified values.
 * Calls from several threads are safe; on one device they run one at a time
 * (they share the device's status word).  Not for use under stream capture
 * (it waits for the stream). */
lowbit_status lowbit_quantize_pack(const void* w, lowbit_dtype w_dtype, int bits, int group, int64_t N,
                                   int64_t K, lowbit_dtype sz_dtype, void* scales, void* zeros,
                                   uint8_t* packed, uint8_t* codes, void* stream);

/* Bytes of workspace that lowbit_linear / lowbit_linear_path can use for the
 * given problem (0 when no schedule needs one).  A call given less than this
 * (including NULL / 0) falls back to a schedule without workspace. */
size_t lowbit_linear_workspace_bytes(int bits, int group, int64_t M, int64_t N, int64_t K,
                                     lowbit_dtype act_dtype);

/* y = x . dequant(packed, scales, zeros)^T (+ bias), enqueued on `stream`
 * (asynchronous: the call returns once the kernels are launched).
 *
 *   x        device, M x K row-major, act_dtype, 16-byte aligned (the
 *            kernels read activations in 16-byte pieces).
 *   packed, scales, zeros   as written by lowbit_quantize_pack with
 *            sz_dtype == act_dtype (or built by the caller in that format);
 *            packed 16-byte aligned, scales and zeros aligned to their
 *            element size.
 *   bias     device, N elements of act_dtype, or NULL for no bias; aligned to
 *            its element size.
 *   y        device, M x N row-major, act_dtype, aligned to its element size.
 *            Overwritten; must not alias any input.
 *   M >= 0 (M == 0 is a no-op that returns LOWBIT_OK; x and y may then be
 *   NULL), N > 0, K > 0,
 *   K % group == 0.
 *   workspace/workspace_bytes: device scratch or NULL/0 (see
 *            lowbit_linear_workspace_bytes).  When non-NULL it must be
 *            256-byte aligned; its contents on entry do not matter and are
 *            overwritten.  Calls that run concurrently must not share one
 *            workspace.
 *
 * Products accumulate in fp32; the bias is added in fp32 and the result is
 * rounded to act_dtype to nearest even.  Determinism: two calls with the
 * same inputs, on the same device model, with the same workspace size (the
 * same K split) and the same schedule overrides (lowbit_tuning.h) give
 * bitwise identical outputs -- no floating-point atomics, and the K split's
 * partial sums are added in a fixed order.  Another workspace size, path or
 * override may choose another schedule, whose results differ in rounding
 * (each accumulated and rounded as stated above). */
lowbit_status lowbit_linear(const void* x, lowbit_dtype act_dtype, const uint8_t* packed,
                            const void* scales, const void* zeros, const void* bias, void* y,
                            int bits, int group, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream);

/* lowbit_linear with an explicit kernel family.  LOWBIT_PATH_QMM with fp32
 * activations returns LOWBIT_ERR_UNSUPPORTED. */
lowbit_status lowbit_linear_path(const void* x, lowbit_dtype act_dtype, const uint8_t* packed,
                                 const void* scales, const void* zeros, const void* bias, void* y,
                                 int bits, int group, int64_t M, int64_t N, int64_t K,
                                 void* workspace, size_t workspace_bytes, lowbit_path path,
                                 void* stream);

/* lowbit_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments and results as lowbit_linear without the workspace: the split-K
 * partial planes of the MFMA schedule live in a device array that the
 * library holds on every GPU it runs on (LOWBIT_NOALLOC_SCRATCH_BYTES =
 * 32 MiB, kept until the process ends).  The call allocates nothing (no
 * hipMalloc, no allocating library routine) and takes the schedule
 * lowbit_linear takes with a workspace of lowbit_linear_workspace_bytes(),
 * so its output is bitwise identical to that call's.  A problem whose
 * schedule needs more than the array holds returns LOWBIT_ERR_WORKSPACE and
 * launches nothing (on a 256-CU device every shape fits).  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give undefined results; calls on one
 * stream run in order and are safe.  The array needs no clearing: each call
 * writes every partial it reads. */
#define LOWBIT_NOALLOC_SCRATCH_BYTES (32u << 20)
lowbit_status lowbit_linear_noalloc(const void* x, lowbit_dtype act_dtype, const uint8_t* packed,
                                    const void* scales, const void* zeros, const void* bias, void* y,
                                    int bits, int group, int64_t M, int64_t N, int64_t K,
                                    void* stream);

/* One linear of a lowbit_linear_multi call (pointers as in lowbit_linear). */
typedef struct lowbit_linear_desc {
  const void* x;          /* device, M x K row-major, act_dtype */
  const uint8_t* packed;  /* device, N x (K*bits/8) bytes, 16-byte aligned */
  const void* scales;     /* device, N x (K/group), act_dtype */
  const void* zeros;      /* device, N x (K/group), act_dtype */
  const void* bias;       /* device, N elements, or NULL */
  void* y;                /* device, M x N row-major, act_dtype; overwritten */
  int64_t N;
  int64_t K;
} lowbit_linear_desc;

#define LOWBIT_MAX_MULTI 8

/* Several independent linears of one bit width, group size, activation
 * dtype and M, computed by the decode kernel in ONE launch: the fused
 * decode step of a layer, e.g. the query/key/value projections or the gate
 * and up projections, which read the same x (the pages' "metal lowbit
 * kernels: qmv_fast optimization" measures whole-model decode, where every
 * linear of a token pays the launch and ramp-up cost; one launch amortizes
 * it).  Each desc has its own x, weights, bias, y, N and K; x may be shared.
 * No y may alias any input of any desc.
 *
 *   count    1 .. LOWBIT_MAX_MULTI (0 is a no-op that returns LOWBIT_OK).
 *   M >= 0   rows of every x (M == 0 is a no-op).  Any M is accepted; the
 *            decode kernel is the one lowbit_linear uses for small M.
 *
 * Every desc is validated as lowbit_linear validates its arguments before
 * anything is launched; on an error nothing is written.  Results are
 * bitwise identical to lowbit_linear_path(..., LOWBIT_PATH_QMV, ...) called
 * on each desc.  Enqueued on `stream`; asynchronous. */
lowbit_status lowbit_linear_multi(const lowbit_linear_desc* descs, int count, lowbit_dtype act_dtype,
                                  int bits, int group, int64_t M, void* stream);

/* ------------------------------------------------------------------------
 * Activation-quantized variant: 8-bit dynamic activations with the groupwise
 * low-bit weights above ("[MPS] Add support for Int4 groupwise quantization":
 * the export mode with 8-bit dynamic activations and 4-bit weights in groups
 * of 32; the page names the mode only, and these conventions fix it):
 *   - each activation row m is quantized at run time, symmetric, with one
 *     fp32 scale: a_m = max_k |x[m, k]| / 127 (correctly rounded fp32
 *     divide), xq[m, k] = clamp(rint_half_even(x[m, k] / a_m), -127, 127)
 *     (fp32 divide); a row whose a_m is 0 gets codes 0; a row holding a NaN
 *     or an infinity gets a_m = NaN and codes 0;
 *   - y[m, n] = a_m * sum_k xq[m, k] * w[n, k] (+ bias[n]), w = s*q + z as
 *     above (any bit width and group size).
 * ---------------------------------------------------------------------- */

/* Quantize activation rows to int8 (the first step of the variant).
 *
 *   x        device, M x K row-major, act_dtype, 16-byte aligned; values are
 *            taken exactly as fp32.
 *   M >= 0 (0 is a no-op), K > 0 and a multiple of 32 (at most 2^30).
 *   xq       device, M x K int8 row-major, 16-byte aligned.  Written.
 *   ascale   device, M fp32, 4-byte aligned.  Written.
 *
 * Asynchronous (enqueued on `stream`); codes and scales are bitwise
 * determined by x.  Non-finite values are not an error: their row is marked
 * by a NaN scale. */
lowbit_status lowbit_quantize_act_i8(const void* x, lowbit_dtype act_dtype, int64_t M, int64_t K,
                                     int8_t* xq, float* ascale, void* stream);

/* y = diag(ascale) . xq . dequant(packed, scales, zeros)^T (+ bias) on the
 * int8 matrix cores: per group the exact int32 sums of xq * q and of xq, each
 * turned into fp32 and scaled by the group's scale and zero; ascale and the
 * bias enter once in fp32 and the result is rounded to dtype to nearest even.
 *
 *   xq, ascale   as written by lowbit_quantize_act_i8 (xq 16-byte aligned).
 *   packed, scales, zeros   as for lowbit_linear, scales and zeros in dtype;
 *            packed 16-byte aligned.
 *   bias     device, N elements of dtype, or NULL.
 *   y        device, M x N row-major, dtype.  Overwritten; must not alias an
 *            input.
 *   dtype    storage type of scales, zeros, bias and y (fp32, fp16, bf16).
 *   M >= 0 (0 is a no-op), N > 0, K % group == 0, M <= 16 * 65535.
 *
 * No workspace, one launch, asynchronous.  Deterministic: no atomics, and
 * every output is summed in one fixed order. */
lowbit_status lowbit_linear_a8(const int8_t* xq, const float* ascale, const uint8_t* packed,
                               const void* scales, const void* zeros, const void* bias, void* y,
                               lowbit_dtype dtype, int bits, int group, int64_t M, int64_t N,
                               int64_t K, void* stream);

/* Static text for a status code. */
const char* lowbit_status_string(lowbit_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* lowbit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H_ */
