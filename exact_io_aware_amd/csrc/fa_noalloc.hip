// Library-owned scratch for the entry points that allocate nothing.
//
// fa_bwd needs a per-row workspace (the row sums D and the base-2
// logsumexp, two float arrays of B*H*N rows) that its caller passes in.
// fa_bwd_noalloc takes it from this file-scope device array instead, so that
// callers which cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc) still get the backward.  The array
// is part of the code object: every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  Calls on one GPU share
// that GPU's copy, so calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr size_t kScratchBytes = (size_t)8 << 20;  // 2^20 rows of D and lse2
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` per device, looked up once per device with
// that device current.  In host code the name `scratch` is only a host-side
// handle for the symbol, never a device address.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace fa
