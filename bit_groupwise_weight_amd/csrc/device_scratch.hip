// Device memory owned by the library, for lowbit_linear_noalloc: callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc) get the split-K partial planes of the MFMA
// schedule from this file-scope array instead of a workspace argument.
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

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace lowbit
