// Device helpers shared by every kernel file (code unpack, RoPE table access, reductions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "commvq_internal.h"

namespace commvq {

// Unpack: byte g of a 16-byte code record (one residual of one token) is the index of group g
// (N = 256, one byte per index). Every kernel that reads codes goes through this function.
__device__ __forceinline__ uint32_t code_index(const uint4& w, int g) {
  const uint32_t word = (g < 4) ? w.x : (g < 8) ? w.y : (g < 12) ? w.z : w.w;
  return (word >> ((g & 3) * 8)) & 0xffu;
}

// 16-byte code record of (kv head, token row, residual r) in a [Hkv][T][R][G] byte array.
__device__ __forceinline__ uint4 load_code_record(const uint8_t* codes, int64_t total_tokens, int kv, int64_t row,
                                                  int R, int r) {
  return *reinterpret_cast<const uint4*>(codes + ((static_cast<int64_t>(kv) * total_tokens + row) * R + r) * 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace commvq
