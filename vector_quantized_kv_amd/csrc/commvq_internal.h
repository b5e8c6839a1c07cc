// Internal declarations shared by the C-ABI front end (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "commvq.h"

namespace commvq {

constexpr int kHeadDim = 128;   // D
constexpr int kPairs = 64;      // RoPE pairs per head
constexpr int kGroups = 16;     // G: code indices per residual per vector
constexpr int kGroupDim = 8;    // W: dims per group (4 RoPE pairs)
constexpr int kCodes = 256;     // N: one byte per index
constexpr int kGqa = 4;         // q heads per KV head
constexpr int kSplitTokens = 2048;  // value_reduce: tokens per (sequence, KV head) work item
constexpr int kPartFloats = 132;    // per (b, q head, split): m, l, 2 pad, o[128]
constexpr int kFineRows = 64;       // RoPE table: fine rows e^{i f theta}, f < 64
// RoPE table sections, in float2 units: fine fp32 [j][f]; fine fp32 group-major [g][h][f][p] with
// j = 4g + 2h + p (16 bytes per (g, h, f): a lane's phases of two pairs); coarse fp32 [c][j]
constexpr int kRopeFine32gOffset = kFineRows * kPairs;
constexpr int kRopeCoarseOffset = kRopeFine32gOffset + kFineRows * kPairs;
constexpr int kAttnMaxBlocksPerWave = 8;  // 64-token blocks per wave per split
constexpr int kCounterBytes = 256;  // attention workspace head: per-(b, kv) arrival counters
constexpr int kAttnMaxSplits = 8192;  // splits per sequence the last-workgroup merge can hold in LDS
// commvq_attn_decode_noalloc: static device scratch per GPU (8 MiB), of which a fixed 64 KiB head holds the
// arrival counters (16384 (sequence, KV head) pairs at most) and the rest the split partials
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(8) << 20;
constexpr size_t kNoAllocCounterBytes = static_cast<size_t>(64) << 10;
constexpr int kCUs = 256;             // compute units the split sizing aims to fill (one workgroup each)

// Bit-packed family (one index per 64 dims): G = 2 groups, N = 64 codewords, 6-bit indices packed per
// token into ceil(6 R G / 32) little-endian 32-bit words, index (r, g) at bit 6 (r G + g).
constexpr int kWideGroups = 2;
constexpr int kWideCodes = 64;
constexpr int kWideBits = 6;
constexpr int kWideMaxResiduals = 32;
constexpr int kWideResPerPass = 8;  // residuals per index window (16 indices, 3 words) and per key pass (8 x 8 KiB)
__host__ __device__ inline int wide_record_words(int R) { return (kWideBits * R * kWideGroups + 31) / 32; }

// Attention workgroup: fp16 storage runs 8 waves (two per SIMD) over two 64 KiB codebook slots; fp32
// storage runs 4 waves over one 128 KiB slot. Either way one workgroup owns a CU's LDS.
inline int attn_waves(int dtype) { return dtype == COMMVQ_F16 ? 8 : 4; }

inline int64_t n_splits_for(int32_t max_len) {
  int64_t s = (static_cast<int64_t>(max_len) + kSplitTokens - 1) / kSplitTokens;
  return s > 0 ? s : 1;
}

// Attention split size: waves x 64 tokens x blocks-per-wave (1..8), chosen so that the grid holds
// about one (sequence, KV head, split) item per CU.
inline int32_t attn_split_tokens(int dtype, int32_t max_len, int32_t batch, int32_t n_kv_heads) {
  const int64_t wg_tokens = 64LL * attn_waves(dtype);
  const int64_t work = static_cast<int64_t>(max_len) * batch * n_kv_heads;
  int64_t blocks_per_wave = (work + kCUs * wg_tokens - 1) / (kCUs * wg_tokens);
  if (blocks_per_wave < 1) blocks_per_wave = 1;
  if (blocks_per_wave > kAttnMaxBlocksPerWave) blocks_per_wave = kAttnMaxBlocksPerWave;
  return static_cast<int32_t>(blocks_per_wave * wg_tokens);
}
inline int64_t attn_n_splits(int32_t max_len, int32_t split_tokens) {
  int64_t s = (static_cast<int64_t>(max_len) + split_tokens - 1) / split_tokens;
  return s > 0 ? s : 1;
}
inline size_t attn_counter_bytes(int32_t batch, int32_t n_kv_heads) {
  size_t b = static_cast<size_t>(batch) * n_kv_heads * sizeof(uint32_t);
  return (b + kCounterBytes - 1) / kCounterBytes * kCounterBytes;
}
inline int64_t rope_coarse_rows(int32_t n_positions) { return (static_cast<int64_t>(n_positions) + 63) / 64; }

struct AttnArgs {
  const void* q;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const void* k_cb;
  const void* v_cb;
  const int64_t* seq_start;
  const int32_t* seq_len;
  int64_t total_tokens;
  int32_t max_len;  // longest sequence the launch was sized for (seq_len is clamped to it)
  const float2* rope;
  int32_t n_splits;
  int32_t split_tokens;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  float scale;
  int32_t n_residuals;   // bit-packed family only
  int32_t record_words;  // bit-packed family only: 32-bit words per token record
  uint32_t* counters;  // [B][Hkv], zero between calls
  float2* part_ml;     // [B][Hq][n_splits]: (m, l) of each split
  float* part_o;       // [B][Hq][n_splits][D]: unnormalised output of each split
  float* out;
};

struct ValueReduceArgs {
  const float* p;
  int32_t p_stride;  // max_len
  const uint8_t* v_codes;
  const void* v_cb;
  const int64_t* seq_start;
  const int32_t* seq_len;
  int64_t total_tokens;
  int32_t n_splits;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  float* part;
};

hipError_t launch_rope_table(double base, int32_t n_positions, float2* table, hipStream_t s);
hipError_t launch_qtable(int dtype, bool packed, int R, int B, int Hq, int Hkv, const void* q, const void* kcb,
                         void* out, hipStream_t s);
hipError_t launch_attn(int dtype, int R, int B, const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f16(int R, int B, const AttnArgs& a, hipStream_t s);
// Device address of this device's static scratch (noalloc.hip); the first call on a device also zeroes its
// counter head on `stream`.
hipError_t noalloc_scratch(void** out, hipStream_t stream);
hipError_t launch_attn_wide(int B, const AttnArgs& a, hipStream_t s);
hipError_t launch_value_reduce(int dtype, bool packed, int R, int B, const ValueReduceArgs& a, float* out,
                               hipStream_t s);
hipError_t launch_encode_greedy(int dtype, int R, int Hkv, const void* x, const void* cb, int64_t n, uint8_t* codes,
                                int64_t total_rows, int64_t first_row, hipStream_t s);
hipError_t launch_encode_greedy_bits(int R, int Hkv, const void* x, const void* cb, int64_t n, uint32_t* words,
                                     int64_t total_rows, int64_t first_row, hipStream_t s);
hipError_t launch_codebook_update(int dtype, int R, int Hkv, const void* x, const uint8_t* codes, int64_t n,
                                  const void* cb_in, void* cb_out, hipStream_t s);
hipError_t launch_codebook_update_bits(int R, int Hkv, const void* x, const uint32_t* words, int64_t n,
                                       const void* cb_in, void* cb_out, hipStream_t s);
hipError_t launch_debug_unpack(int R, int Hkv, int64_t total_tokens, const uint8_t* codes, int32_t* out,
                               hipStream_t s);
hipError_t launch_debug_unpack_bits(int R, int Hkv, int64_t total_tokens, const uint32_t* words, int32_t* out,
                                    hipStream_t s);

}  // namespace commvq
