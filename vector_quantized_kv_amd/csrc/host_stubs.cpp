// Host-only stand-ins for the device side of libcommvq, for the sanitizer build of the C ABI's host code
// (argument checks, workspace sizing, error reporting). Every launch reports hipErrorNoDevice, as the real
// library does on a machine without a GPU, so a call that passes its checks returns COMMVQ_EHIP and no
// kernel, device memory or HIP runtime is involved. Never part of libcommvq.so.
#include "commvq_internal.h"

namespace commvq {

hipError_t launch_rope_table(double, int32_t, float2*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_qtable(int, bool, int, int, int, int, const void*, const void*, void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attn(int, int, int, const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_f16(int, int, const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void**, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_wide(int, const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_value_reduce(int, bool, int, int, const ValueReduceArgs&, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_encode_greedy(int, int, int, const void*, const void*, int64_t, uint8_t*, int64_t, int64_t,
                                hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_encode_greedy_bits(int, int, const void*, const void*, int64_t, uint32_t*, int64_t, int64_t,
                                     hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_codebook_update(int, int, int, const void*, const uint8_t*, int64_t, const void*, void*,
                                  hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_codebook_update_bits(int, int, const void*, const uint32_t*, int64_t, const void*, void*,
                                       hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_debug_unpack(int, int, int64_t, const uint8_t*, int32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_debug_unpack_bits(int, int, int64_t, const uint32_t*, int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace commvq

// The one HIP runtime call of the host code (its error path), without the runtime.
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "no GPU (host-only build)"; }
