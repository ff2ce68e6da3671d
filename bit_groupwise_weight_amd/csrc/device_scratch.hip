// Device memory owned by the library: the scratch array of
// lowbit_linear_noalloc -- callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc) get the
// split-K partial planes of the MFMA schedule from it instead of a workspace
// argument -- and the quantizer's status flags.
//
// Every device the library runs on holds its own copy of the array from the
// moment the code object is loaded there until the process ends.  In host
// code the array's name is only a host-side stand-in: its device address is
// taken once per device with hipGetSymbolAddress (with that device current)
// and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace lowbit {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
// The quantizer's two status flags (non-finite weight, scale or zero out of
// range), likewise one copy per device.
static __device__ __align__(256) int quant_status[2];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
void* g_status_ptr[kMaxScratchDevices] = {};

// Device address of `symbol` on the current device, looked up once per
// device (with that device current) and kept in `cache`.
hipError_t device_address(const void* symbol, void* (&cache)[kMaxScratchDevices], void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, symbol);
    if (e != hipSuccess) return e;
    cache[dev] = p;
  }
  *out = cache[dev];
  return hipSuccess;
}
}  // namespace

hipError_t noalloc_scratch(void** out) {
  return device_address(HIP_SYMBOL(scratch), g_scratch_ptr, out);
}

hipError_t quant_status_words(int** out) {
  void* p = nullptr;
  const hipError_t e = device_address(HIP_SYMBOL(quant_status), g_status_ptr, &p);
  *out = static_cast<int*>(p);
  return e;
}

}  // namespace lowbit
