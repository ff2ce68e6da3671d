// Measurement instruments for the decode kernel's roofline (the library
// liblowbit_probe.so, C ABI in include/lowbit_probe.h): what a plain
// streaming read of the same bytes achieves in one launch, and the latency of
// one dependent load from HBM.  Neither is part of the layer; the benchmark
// reports them beside the decode timings, because at decode sizes (a few MB)
// launch and memory latency, not bandwidth, bound a single kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "lowbit_probe.h"

namespace lowbit {

// Reads n16 16-byte words, LPT independent loads per thread per round
// (grid-stride), and folds them into one word that is stored only if it
// matches a constant, which keeps every load live without a store per
// thread.
template <int LPT>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  uint32_t acc = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += LPT * stride) {
    uint4 v[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int64_t k = i + j * stride;
      v[j] = k < n16 ? src[k] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LPT; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, int loads_per_thread, uint32_t* sink,
                              hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = 256LL * loads_per_thread;
  const unsigned blocks = static_cast<unsigned>(std::max<int64_t>(1, (n16 + per_block - 1) / per_block));
  const uint4* p = static_cast<const uint4*>(src);
  switch (loads_per_thread) {
    case 1: stream_read_kernel<1><<<blocks, 256, 0, s>>>(p, n16, sink); break;
    case 2: stream_read_kernel<2><<<blocks, 256, 0, s>>>(p, n16, sink); break;
    case 4: stream_read_kernel<4><<<blocks, 256, 0, s>>>(p, n16, sink); break;
    case 8: stream_read_kernel<8><<<blocks, 256, 0, s>>>(p, n16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One lane follows `hops` links of a chain (i <- chain[i]) from `start`;
// every load depends on the previous one.  Links are clamped to the chain,
// so any chain contents stay in bounds.  The end index is stored so the
// chain cannot be skipped.
__global__ __launch_bounds__(64) void chase_kernel(const uint32_t* __restrict__ chain, uint32_t last,
                                                   int hops, uint32_t start, uint32_t* out) {
  if (threadIdx.x != 0) return;
  uint32_t i = start;
  for (int h = 0; h < hops; ++h) i = min(__builtin_nontemporal_load(chain + i), last);
  out[0] = i;
}

hipError_t launch_chase(const uint32_t* chain, int64_t chain_len, int hops, uint32_t start,
                        uint32_t* out, hipStream_t s) {
  chase_kernel<<<1, 64, 0, s>>>(chain, static_cast<uint32_t>(chain_len - 1), hops, start, out);
  return hipGetLastError();
}

}  // namespace lowbit

namespace {
thread_local std::string g_probe_error;

lowbit_status probe_fail(lowbit_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lowbit_status probe_fail(lowbit_status st, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_probe_error = buf;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
}  // namespace

extern "C" {

lowbit_status lowbit_probe_stream_read(const void* src, size_t bytes, int loads_per_thread,
                                       uint32_t* sink, void* stream) {
  g_probe_error.clear();
  if (!src || !sink) return probe_fail(LOWBIT_ERR_INVALID_ARG, "NULL src or sink");
  if (bytes == 0 || bytes % 16 != 0 || bytes > (size_t{1} << 40))
    return probe_fail(LOWBIT_ERR_INVALID_ARG, "bytes=%zu must be a positive multiple of 16", bytes);
  if (loads_per_thread != 1 && loads_per_thread != 2 && loads_per_thread != 4 && loads_per_thread != 8)
    return probe_fail(LOWBIT_ERR_INVALID_ARG, "loads_per_thread=%d not one of 1/2/4/8", loads_per_thread);
  if (!aligned(src, 16) || !aligned(sink, 4)) return probe_fail(LOWBIT_ERR_MISALIGNED, "src/sink alignment");
  const hipError_t e = lowbit::launch_stream_read(src, static_cast<int64_t>(bytes), loads_per_thread,
                                                  sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOWBIT_OK : probe_fail(LOWBIT_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
}

lowbit_status lowbit_probe_chase(const uint32_t* chain, int64_t chain_len, int hops, uint32_t start,
                                 uint32_t* out, void* stream) {
  g_probe_error.clear();
  if (!chain || !out) return probe_fail(LOWBIT_ERR_INVALID_ARG, "NULL chain or out");
  if (chain_len < 1 || chain_len > (int64_t{1} << 32))
    return probe_fail(LOWBIT_ERR_INVALID_ARG, "chain_len=%lld not in 1..2^32", (long long)chain_len);
  if (hops < 0 || hops > (1 << 24)) return probe_fail(LOWBIT_ERR_INVALID_ARG, "hops=%d not in 0..2^24", hops);
  if (static_cast<int64_t>(start) >= chain_len)
    return probe_fail(LOWBIT_ERR_INVALID_ARG, "start=%u past the chain", start);
  if (!aligned(chain, 4) || !aligned(out, 4)) return probe_fail(LOWBIT_ERR_MISALIGNED, "chain/out alignment");
  const hipError_t e = lowbit::launch_chase(chain, chain_len, hops, start, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOWBIT_OK : probe_fail(LOWBIT_ERR_HIP, "chase launch: %s", hipGetErrorString(e));
}

const char* lowbit_probe_last_error(void) { return g_probe_error.c_str(); }

}  // extern "C"
