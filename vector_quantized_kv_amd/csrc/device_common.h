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

// Bounds of sequence b as every kernel uses them. seq_start and seq_len live in device memory, where the
// host cannot check them, so they are clamped: the start into [0, total_tokens], the length into
// [0, min(max_len, total_tokens - start)]. Descriptors within the documented bounds pass unchanged; any
// other one still reads only rows of the code arrays, positions of the RoPE table and splits of the
// workspace that exist. Loaded before any other memory operation of a kernel, they stay scalar.
struct SeqBounds {
  int64_t start;
  int len;
};
__device__ __forceinline__ SeqBounds seq_bounds(const int64_t* seq_start, const int32_t* seq_len, int b,
                                                int32_t max_len, int64_t total_tokens) {
  const int64_t s = min(max(seq_start[b], static_cast<int64_t>(0)), total_tokens);
  const int64_t L = min(min(static_cast<int64_t>(max(seq_len[b], 0)), static_cast<int64_t>(max_len)), total_tokens - s);
  return {s, static_cast<int>(L)};
}

// 16-byte code record of (kv head, token row, residual r) in a [Hkv][R][T][G] byte array.
__device__ __forceinline__ uint4 load_code_record(const uint8_t* codes, int64_t total_tokens, int kv, int64_t row,
                                                  int R, int r) {
  return *reinterpret_cast<const uint4*>(codes + ((static_cast<int64_t>(kv) * R + r) * total_tokens + row) * 16);
}

// Bit-packed records (one index per 64 dims, N = 64): a token's R x 2 six-bit indices form one
// little-endian bitstream of 32-bit words, index (r, g) at bit 6 (2 r + g). Word w of every token of a KV head
// sits in plane w ([Hkv][words][T]), so a token's words are T apart. Kernels read the stream in windows of
// kWideResPerPass residuals: window c is the 96 bits of words 3 c .. 3 c + 2 (words past the record are
// read as its last word; the fields they would hold lie past bit 12 R and are never used).
__device__ __forceinline__ int packed_window_word(int c) { return (kWideBits * kWideGroups * kWideResPerPass * c) >> 5; }
static_assert(kWideBits * kWideGroups * kWideResPerPass == 96, "a window is three whole words");
// Index F of a window from its words (x0, x1, x2); F = 2 rho + g for residual kWideResPerPass * c + rho,
// group g.
template <int F>
__device__ __forceinline__ uint32_t packed_index(uint32_t x0, uint32_t x1, uint32_t x2) {
  constexpr int bit = kWideBits * F, wi = bit >> 5, sh = bit & 31;
  constexpr uint32_t mask = (1u << kWideBits) - 1;
  static_assert(wi < 3, "inside the window");
  const uint32_t lo = wi == 0 ? x0 : (wi == 1 ? x1 : x2);
  if constexpr (sh + kWideBits <= 32) {
    return (lo >> sh) & mask;
  } else {
    const uint32_t hi = wi == 0 ? x1 : x2;
    return __builtin_amdgcn_alignbit(hi, lo, sh) & mask;
  }
}
// Index (r, g) of one token record whose words are `plane` apart, read field by field (the codebook tools;
// the attention kernel reads whole windows). A field that crosses a word boundary takes its high bits from
// the next word, which is then still inside the record (the field ends at or before bit 12 R).
__device__ __forceinline__ uint32_t packed_field(const uint32_t* rec, int64_t plane, int r, int g) {
  const int bit = kWideBits * (kWideGroups * r + g), w = bit >> 5, sh = bit & 31;
  uint32_t v = rec[w * plane] >> sh;
  if (sh > 32 - kWideBits) v |= rec[(w + 1) * plane] << (32 - sh);
  return v & ((1u << kWideBits) - 1);
}

// row_ror DPP: lane l of each 16-lane row reads lane (l + n) mod 16 of the same row. Every source lane
// exists, so bound_ctrl is irrelevant to the result; setting it lets the compiler fold the move into the
// consuming add or max.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf,
                                                               true));
}
// Half-wave swap reductions of two registers x, y into one.
// swap32_add: lanes 0..31 get x[l] + x[l + 32], lanes 32..63 get y[l - 32] + y[l].
// swap16_add: per 16-lane row, row 0 gets x row 0 + x row 1, row 1 gets y rows 0 + 1, row 2 gets
// x rows 2 + 3, row 3 gets y rows 2 + 3 (lane offsets within the row are kept).
__device__ __forceinline__ float swap32_add(float x, float y) {
  const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  const unsigned s0 = s[0], s1 = s[1];  // (bit-casting a vector element directly reads element 0)
  return __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
}
__device__ __forceinline__ float swap16_add(float x, float y) {
  const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  const unsigned s0 = s[0], s1 = s[1];  // (bit-casting a vector element directly reads element 0)
  return __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wave-wide reductions (all 64 lanes active): four row_ror DPP steps leave each 16-lane row's result in
// every lane of the row; the four row results are then read as scalars. The result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<1>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

}  // namespace commvq
