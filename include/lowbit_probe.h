/*
 * lowbit_probe.h -- measurement instruments of the benchmark, built as their
 * own library (liblowbit_probe.so), not part of the layer.
 *
 * The decode kernel reads a few MB per call, where launch and memory latency
 * rather than bandwidth bound any single kernel.  These two calls measure
 * that floor on the running device so a benchmark can report the decode
 * kernel against it.  Statuses and lowbit_last_error() follow lowbit.h.
 */
#ifndef LOWBIT_PROBE_H_
#define LOWBIT_PROBE_H_

#include "lowbit.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a positive multiple of 16, src 16-byte aligned) from device
 * memory with plain 16-byte loads, loads_per_thread (1, 2, 4 or 8) per
 * thread per round, in one launch of 256-thread blocks, and discards the data
 * (`sink`, one device word, is written only if the data fold to a fixed
 * constant).  Enqueued on `stream`. */
lowbit_status lowbit_probe_stream_read(const void* src, size_t bytes, int loads_per_thread,
                                       uint32_t* sink, void* stream);

/* One lane follows `hops` (0 .. 2^24) dependent links i <- chain[i] of the
 * device array chain[0 .. chain_len) from index `start`, each link clamped to
 * chain_len - 1 (any contents are safe), and writes the final index to the
 * device word `out`.  With links that point to distinct cache lines outside
 * every cache, the time per hop is the latency of one load from HBM.
 * Enqueued on `stream`. */
lowbit_status lowbit_probe_chase(const uint32_t* chain, int64_t chain_len, int hops, uint32_t start,
                                 uint32_t* out, void* stream);

/* Detail of the last failure of a probe call on the calling thread. */
const char* lowbit_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_PROBE_H_ */
