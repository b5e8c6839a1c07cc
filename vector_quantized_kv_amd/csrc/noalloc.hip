// Static device scratch for commvq_attn_decode_noalloc, the attention entry point that allocates nothing.
//
// The array lives in the library's code object: every GPU the library runs on holds its own copy, at its own
// address, from the first call on that device until the process ends. Host code never passes the array's
// name to a kernel (in host code it is only a stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
//
// Layout (fixed, so that calls of any shape agree on where the arrival counters are):
//   [0, kNoAllocCounterBytes)              arrival counters, one per (sequence, KV head); zero between calls
//   [kNoAllocCounterBytes, kNoAllocScratchBytes)   split partials (m, l) and o[128] of the current call
// Every call on a device shares that device's array, so calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "commvq_internal.h"

namespace commvq {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [&] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g_status[dev] != hipSuccess) return;
    g_scratch[dev] = p;
    // the counters must start at zero (every completed call leaves them zero again); a fill kernel rather than
    // a memset, so that a call made under graph capture records only kernels
    constexpr int kWords = kNoAllocCounterBytes / 4;
    zero_words_kernel<<<dim3((kWords + 255) / 256), dim3(256), 0, stream>>>(static_cast<uint32_t*>(p), kWords);
    g_status[dev] = hipGetLastError();
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace commvq
