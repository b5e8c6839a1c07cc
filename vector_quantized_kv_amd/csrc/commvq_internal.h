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
constexpr int kSplitTokens = 1024;  // tokens per (sequence, KV head) work item
constexpr int kPartFloats = 132;    // per (b, q head, split): m, l, 2 pad, o[128]
constexpr int kFineRows = 64;       // RoPE table: fine rows e^{i f theta}, f < 64

inline int64_t n_splits_for(int32_t max_len) {
  int64_t s = (static_cast<int64_t>(max_len) + kSplitTokens - 1) / kSplitTokens;
  return s > 0 ? s : 1;
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
  const float2* rope;
  int32_t n_splits;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  float scale;
  float* part;
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
hipError_t launch_qtable(int dtype, int R, int B, int Hq, int Hkv, const void* q, const void* kcb, void* out,
                         hipStream_t s);
hipError_t launch_attn(int dtype, int R, int B, const AttnArgs& a, float* out, hipStream_t s);
hipError_t launch_value_reduce(int dtype, int R, int B, const ValueReduceArgs& a, float* out, hipStream_t s);
hipError_t launch_debug_unpack(int R, int Hkv, int64_t total_tokens, const uint8_t* codes, int32_t* out,
                               hipStream_t s);

}  // namespace commvq
