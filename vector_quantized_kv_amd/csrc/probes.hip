// Measurement probes for the benchmark (declared in commvq_probes.h): a streaming HBM read, the LDS
// random-gather throughput and the throughput of random 64-bit LDS atomic adds. Not part of the attention
// path; built into libcommvq_probes.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "commvq_probes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kNever = 0x9e3779b9u;  // the folded value is written only if it equals this

__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // four independent loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == kNever) sink[0] = v;
}

constexpr int kProbeWaves = 8;
constexpr int kRows = 256, kGroupBytes = kRows * 16, kTableBytes = 16 * kGroupBytes;
constexpr int kLdsBytes = 160 * 1024;  // one workgroup per CU

__global__ void __launch_bounds__(kProbeWaves * 64) lds_gather_kernel(int iters, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  const int tid = threadIdx.x;
  for (int i = tid; i < kTableBytes / 16; i += kProbeWaves * 64)
    reinterpret_cast<u32x4*>(lds)[i] = (u32x4){static_cast<uint32_t>(i), static_cast<uint32_t>(3 * i),
                                               static_cast<uint32_t>(5 * i), static_cast<uint32_t>(7 * i)};
  __syncthreads();
  // a random row per lane and group (a different generator state per lane, workgroup and group)
  uint32_t x = 0x12345678u ^ (static_cast<uint32_t>(tid) * 0x9e3779b1u) ^ (blockIdx.x * 0x85ebca6bu);
  uint32_t off[16];
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    x = x * 1664525u + 1013904223u;
    off[g] = (x >> 24) * 16;
  }
  for (int it = 0; it < iters; ++it) {
    // every iteration reads other rows of the same groups (the row offsets flipped by the iteration number)
    const uint32_t flip = static_cast<uint32_t>(it & 15) << 4;
    u32x4 r[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) r[g] = *reinterpret_cast<const u32x4*>(lds + g * kGroupBytes + (off[g] ^ flip));
    // the rows are consumed by an empty asm statement: no arithmetic competes with the reads
#pragma unroll
    for (int g = 0; g < 16; ++g) asm volatile("" ::"v"(r[g]));
  }
  if (iters == -1) sink[0] = kNever;  // (never: iters >= 1) keeps sink an argument of the kernel
}

// Random 64-bit LDS adds into bins laid out as the bit-packed attention kernel's value bins: 42 units
// (R = 21 residuals x 2 groups) of [2 head pairs][64 codewords] 64-bit words, 43 KiB; per unit every lane adds
// to the same random codeword of both head pairs (two wave instructions). The bins' total is written to sink
// (so the adds are kept), and it equals 2 x 42 x iters x 512 per workgroup.
constexpr int kBinUnits = 42;

__global__ void __launch_bounds__(kProbeWaves * 64) lds_bin_add_kernel(int iters, unsigned long long* sink) {
  // 160 KiB, of which the bins use the first 43 KiB: one workgroup per CU, as in the attention kernel
  __shared__ unsigned long long bins[kLdsBytes / 8];
  static_assert(kBinUnits * 2 * 64 * 8 <= kLdsBytes, "the bins fit the array");
  const int tid = threadIdx.x;
  for (int i = tid; i < kBinUnits * 2 * 64; i += kProbeWaves * 64) bins[i] = 0;
  __syncthreads();
  uint32_t x = 0x2545f491u ^ (static_cast<uint32_t>(tid) * 0x9e3779b1u) ^ (blockIdx.x * 0x85ebca6bu);
  for (int it = 0; it < iters; ++it) {
#pragma unroll 6
    for (int u = 0; u < kBinUnits; ++u) {
      x = x * 1664525u + 1013904223u;
      unsigned long long* b = bins + u * 128 + (x >> 26);
      __hip_atomic_fetch_add(b, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_add(b + 64, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  unsigned long long t = 0;
  for (int i = tid; i < kBinUnits * 2 * 64; i += kProbeWaves * 64) t += bins[i];
  atomicAdd(sink, t);
}

}  // namespace

extern "C" {

int commvq_probe_read_stream(const void* buf, size_t bytes, int blocks, void* sink, void* stream) {
  if (!buf || !sink || blocks < 1 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return static_cast<int>(hipErrorInvalidValue);
  read_stream_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(buf), bytes / 16,
                                                                          static_cast<uint32_t*>(sink));
  return static_cast<int>(hipGetLastError());
}

int commvq_probe_lds_bin_add(int iters, int blocks, void* sink, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return static_cast<int>(hipErrorInvalidValue);
  lds_bin_add_kernel<<<blocks, kProbeWaves * 64, 0, static_cast<hipStream_t>(stream)>>>(
      iters, static_cast<unsigned long long*>(sink));
  return static_cast<int>(hipGetLastError());
}

int commvq_probe_lds_gather(int iters, int blocks, void* sink, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return static_cast<int>(hipErrorInvalidValue);
  lds_gather_kernel<<<blocks, kProbeWaves * 64, 0, static_cast<hipStream_t>(stream)>>>(iters,
                                                                                     static_cast<uint32_t*>(sink));
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
