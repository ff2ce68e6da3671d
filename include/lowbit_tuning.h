/*
 * lowbit_tuning.h -- overrides of the automatic kernel-schedule choices of
 * liblowbit.so, for tests and benchmarks (not part of the layer).
 *
 * By default every schedule choice (decode block size and register
 * variant; MFMA row tiles, column tiles, waves, K groups and the block
 * target of the K split) is made from the problem shape and the device
 * alone; the library reads no environment variables.  An override applies
 * to every later call in the process, on every device, until set back to
 * 0.  Results stay within the same tolerance of the exact product under any
 * override; only the summation order, and therefore the last bits, may
 * change.  Setting an override while other threads call the library is
 * allowed (each call reads each value once) but makes which calls see it
 * unspecified.
 */
#ifndef LOWBIT_TUNING_H_
#define LOWBIT_TUNING_H_

#include "lowbit.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lowbit_tuning_key {
  LOWBIT_TUNE_QMV_BLOCK = 0,    /* decode threads per block: 64, 128 or 256         */
  LOWBIT_TUNE_QMV_VARIANT = 1,  /* decode register variant + 1 (1..4), one x row    */
  LOWBIT_TUNE_QMM_BLOCKS = 2,   /* MFMA path: block target of the K split           */
  LOWBIT_TUNE_QMM_MTT = 3,      /* MFMA path: at most this many 16-row tiles        */
  LOWBIT_TUNE_QMM_KGROUPS = 4,  /* fp16 MFMA kernel: 1 or 2 K groups                */
  LOWBIT_TUNE_QMM_NT = 5,       /* fp16 MFMA kernel: 1 or 2 column tiles per wave   */
  LOWBIT_TUNE_QMM_WAVES = 6,    /* fp16 MFMA kernel, one K group: 4 or 8 waves      */
  LOWBIT_TUNE_QMM_RGROUPS = 7,  /* bf16 MFMA kernel: 1 or 2 row groups of 4 waves   */
  LOWBIT_TUNE_QMM_SMALL_M = 8,  /* fp16: largest M of the small-M MFMA kernel (1-16;
                                   1 = not used)                                    */
  LOWBIT_TUNE_A8_MTT = 9,       /* int8-activation linear: 16-row tiles per block
                                   (1, 2 or 4)                                      */
  LOWBIT_TUNE_A8_NT = 10,       /* int8-activation linear: 16-column tiles per wave
                                   (1 or 2)                                         */
  LOWBIT_TUNE_COUNT = 11
} lowbit_tuning_key;

/* Set (value > 0) or clear (value == 0) one override.  LOWBIT_ERR_INVALID_ARG
 * for an unknown key or a negative value; values a schedule cannot use are
 * ignored by it. */
lowbit_status lowbit_set_tuning(lowbit_tuning_key key, int value);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_TUNING_H_ */
