// C-ABI front end of libcommvq: host-side argument checks, workspace sizing and launches.
// Every check runs before any HIP call, so a rejected call has no side effects.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>

#include "commvq_internal.h"

using namespace commvq;

namespace {

thread_local char g_detail[512];  // detail of this thread's last failing call (a fixed buffer: nothing allocates)

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_detail[0] = '\0';
  return COMMVQ_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(COMMVQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool packed_family(const commvq_dims* d) { return d->n_groups == kWideGroups && d->n_codes == kWideCodes; }

// Shape checks shared by every entry point. Two index layouts are implemented: one byte per index
// (n_groups 16, n_codes 256, R 1 or 2, fp16 or fp32) and bit-packed records (n_groups 2, n_codes 64,
// R 1 .. kWideMaxResiduals, fp16).
int check_dims(const commvq_dims* d) {
  if (!d) return fail(COMMVQ_EINVAL, "dims is NULL");
  if (d->batch < 1) return fail(COMMVQ_EINVAL, "batch = %d must be >= 1", d->batch);
  if (d->n_kv_heads < 1 || d->n_q_heads < 1)
    return fail(COMMVQ_EINVAL, "n_q_heads = %d and n_kv_heads = %d must be >= 1", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(COMMVQ_EINVAL, "n_q_heads = %d is not a multiple of n_kv_heads = %d", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads / d->n_kv_heads != kGqa)
    return fail(COMMVQ_EUNSUPPORTED, "q heads per KV head = %d; only %d is implemented",
                d->n_q_heads / d->n_kv_heads, kGqa);
  if (d->head_dim != kHeadDim) return fail(COMMVQ_EUNSUPPORTED, "head_dim = %d; only %d is implemented", d->head_dim, kHeadDim);
  if (d->n_residuals < 1) return fail(COMMVQ_EINVAL, "n_residuals = %d must be >= 1", d->n_residuals);
  if (d->dtype != COMMVQ_F16 && d->dtype != COMMVQ_F32) return fail(COMMVQ_EINVAL, "dtype = %d is not a commvq_dtype", d->dtype);
  if (packed_family(d)) {
    if (d->n_residuals > kWideMaxResiduals)
      return fail(COMMVQ_EUNSUPPORTED, "n_residuals = %d; the bit-packed layout implements 1 .. %d", d->n_residuals,
                  kWideMaxResiduals);
    if (d->dtype != COMMVQ_F16) return fail(COMMVQ_EUNSUPPORTED, "the bit-packed layout implements fp16 codebooks only");
  } else {
    if (d->n_groups != kGroups || d->n_codes != kCodes)
      return fail(COMMVQ_EUNSUPPORTED, "(n_groups, n_codes) = (%d, %d); only (%d, %d) and (%d, %d) are implemented",
                  d->n_groups, d->n_codes, kGroups, kCodes, kWideGroups, kWideCodes);
    if (d->n_residuals > 2)
      return fail(COMMVQ_EUNSUPPORTED, "n_residuals = %d; the byte layout implements 1 and 2", d->n_residuals);
  }
  if (!(d->rope_base > 1.0)) return fail(COMMVQ_EINVAL, "rope_base = %g must be > 1", d->rope_base);
  if (!std::isfinite(d->softmax_scale) || d->softmax_scale == 0.f)
    return fail(COMMVQ_EINVAL, "softmax_scale must be finite and non-zero");
  return COMMVQ_OK;
}

size_t rope_bytes(int32_t n_positions) {
  return (static_cast<size_t>(kRopeCoarseOffset) + static_cast<size_t>(rope_coarse_rows(n_positions)) * kPairs) *
         sizeof(float2);
}

size_t part_bytes(const commvq_dims* d, int32_t max_len) {
  return static_cast<size_t>(d->batch) * d->n_q_heads * n_splits_for(max_len) * kPartFloats * sizeof(float);
}

// attention workspace: [arrival counters, padded to 256 B][(m, l) per (b, q head, split), padded to 256 B]
// [o[D] per (b, q head, split)]
struct AttnWs {
  size_t ml_offset, o_offset, bytes;
};
AttnWs attn_ws(const commvq_dims* d, int32_t max_len) {
  const int32_t S = attn_split_tokens(d->dtype, max_len, d->batch, d->n_kv_heads);
  const size_t items = static_cast<size_t>(d->batch) * d->n_q_heads * attn_n_splits(max_len, S);
  AttnWs w;
  w.ml_offset = attn_counter_bytes(d->batch, d->n_kv_heads);
  w.o_offset = w.ml_offset + (items * sizeof(float2) + 255) / 256 * 256;
  w.bytes = w.o_offset + items * kHeadDim * sizeof(float);
  return w;
}
size_t attn_ws_bytes(const commvq_dims* d, int32_t max_len) { return attn_ws(d, max_len).bytes; }


// Argument checks shared by both attention entry points (every check runs before any HIP call).
int check_attn_args(const commvq_dims* d, const void* q, const uint8_t* k_codes, const uint8_t* v_codes,
                    const void* k_codebook, const void* v_codebook, const int64_t* seq_start, const int32_t* seq_len,
                    int32_t max_len, int64_t total_tokens, const void* rope_table, int32_t rope_positions,
                    const float* out) {
  if (int st = check_dims(d)) return st;
  if (!q || !k_codes || !v_codes || !k_codebook || !v_codebook || !seq_start || !seq_len || !rope_table || !out)
    return fail(COMMVQ_EINVAL, "a required pointer is NULL");
  if (max_len < 0) return fail(COMMVQ_EINVAL, "max_len = %d must be >= 0", max_len);
  if (total_tokens < 0) return fail(COMMVQ_EINVAL, "total_tokens = %lld must be >= 0", (long long)total_tokens);
  if (max_len > 0 && total_tokens < 1) return fail(COMMVQ_EINVAL, "total_tokens must be >= 1 when max_len > 0");
  if (rope_positions < max_len)
    return fail(COMMVQ_EINVAL, "rope_positions = %d < max_len = %d", rope_positions, max_len);
  if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(rope_table) || !aligned16(k_codebook) ||
      !aligned16(v_codebook))
    return fail(COMMVQ_EINVAL, "k_codes, v_codes, both codebooks and rope_table must be 16-byte aligned");
  const int32_t split_tokens = attn_split_tokens(d->dtype, max_len, d->batch, d->n_kv_heads);
  if (attn_n_splits(max_len, split_tokens) > kAttnMaxSplits)
    return fail(COMMVQ_EUNSUPPORTED, "max_len = %d needs more than %d splits of %d tokens", max_len, kAttnMaxSplits,
                split_tokens);
  return COMMVQ_OK;
}

// Launch of either layout's attention kernel with the workspace regions given (arrival counters, (m, l) and
// o partials); the arguments have been checked.
int launch_attn_decode(const commvq_dims* d, const void* q, const uint8_t* k_codes, const uint8_t* v_codes,
                       const void* k_codebook, const void* v_codebook, const int64_t* seq_start,
                       const int32_t* seq_len, int32_t max_len, int64_t total_tokens, const void* rope_table,
                       void* counters, void* part_ml, void* part_o, float* out, void* stream) {
  const int32_t split_tokens = attn_split_tokens(d->dtype, max_len, d->batch, d->n_kv_heads);
  AttnArgs a;
  a.q = q;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_cb = k_codebook;
  a.v_cb = v_codebook;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.total_tokens = total_tokens;
  a.max_len = max_len;
  a.rope = static_cast<const float2*>(rope_table);
  a.split_tokens = split_tokens;
  a.n_splits = static_cast<int32_t>(attn_n_splits(max_len, split_tokens));
  a.n_q_heads = d->n_q_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.scale = d->softmax_scale;
  a.n_residuals = d->n_residuals;
  a.record_words = wide_record_words(d->n_residuals);
  a.counters = static_cast<uint32_t*>(counters);
  a.part_ml = static_cast<float2*>(part_ml);
  a.part_o = static_cast<float*>(part_o);
  a.out = out;
  if (packed_family(d))
    return hip_status(launch_attn_wide(d->batch, a, static_cast<hipStream_t>(stream)), "attn_decode launch");
  return hip_status(launch_attn(d->dtype, d->n_residuals, d->batch, a, static_cast<hipStream_t>(stream)),
                    "attn_decode launch");
}

}  // namespace

extern "C" {

const char* commvq_status_string(int status) {
  switch (status) {
    case COMMVQ_OK: return "ok";
    case COMMVQ_EINVAL: return "invalid argument";
    case COMMVQ_EUNSUPPORTED: return "unsupported configuration";
    case COMMVQ_EWORKSPACE: return "workspace too small";
    case COMMVQ_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* commvq_last_error_detail(void) { return g_detail; }

size_t commvq_rope_table_size(const commvq_dims* d, int32_t n_positions) {
  if (check_dims(d) != COMMVQ_OK || n_positions < 1) return 0;
  return rope_bytes(n_positions);
}

int commvq_rope_table(const commvq_dims* d, int32_t n_positions, void* table, size_t table_bytes, void* stream) {
  if (int st = check_dims(d)) return st;
  if (n_positions < 1) return fail(COMMVQ_EINVAL, "n_positions = %d must be >= 1", n_positions);
  if (!table) return fail(COMMVQ_EINVAL, "table is NULL");
  if (table_bytes < rope_bytes(n_positions))
    return fail(COMMVQ_EWORKSPACE, "table_bytes = %zu < %zu", table_bytes, rope_bytes(n_positions));
  if (!aligned16(table)) return fail(COMMVQ_EINVAL, "table must be 16-byte aligned");
  return hip_status(launch_rope_table(d->rope_base, n_positions, static_cast<float2*>(table),
                                      static_cast<hipStream_t>(stream)),
                    "rope_table launch");
}

int commvq_qcodebook_table(const commvq_dims* d, const void* q, const void* k_codebook, void* table, void* stream) {
  if (int st = check_dims(d)) return st;
  if (!q || !k_codebook || !table) return fail(COMMVQ_EINVAL, "q, k_codebook and table must be non-NULL");
  if (!aligned16(k_codebook) || !aligned16(table))
    return fail(COMMVQ_EINVAL, "k_codebook and table must be 16-byte aligned");
  return hip_status(launch_qtable(d->dtype, packed_family(d), d->n_residuals, d->batch, d->n_q_heads, d->n_kv_heads,
                                  q, k_codebook, table, static_cast<hipStream_t>(stream)),
                    "qcodebook_table launch");
}

size_t commvq_attn_decode_workspace_size(const commvq_dims* d, int32_t max_len) {
  if (check_dims(d) != COMMVQ_OK || max_len < 0) return 0;
  return attn_ws_bytes(d, max_len);
}

int commvq_attn_decode(const commvq_dims* d, const void* q, const uint8_t* k_codes, const uint8_t* v_codes,
                       const void* k_codebook, const void* v_codebook, const int64_t* seq_start,
                       const int32_t* seq_len, int32_t max_len, int64_t total_tokens, const void* rope_table,
                       int32_t rope_positions, void* workspace, size_t ws_bytes, float* out, void* stream) {
  if (int st = check_attn_args(d, q, k_codes, v_codes, k_codebook, v_codebook, seq_start, seq_len, max_len,
                               total_tokens, rope_table, rope_positions, out))
    return st;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(COMMVQ_EINVAL, "workspace must be 256-byte aligned");
  const size_t need = attn_ws_bytes(d, max_len);
  if (!workspace || ws_bytes < need) return fail(COMMVQ_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  const AttnWs w = attn_ws(d, max_len);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  return launch_attn_decode(d, q, k_codes, v_codes, k_codebook, v_codebook, seq_start, seq_len, max_len,
                            total_tokens, rope_table, ws, ws + w.ml_offset, ws + w.o_offset, out, stream);
}

int commvq_attn_decode_noalloc(const commvq_dims* d, const void* q, const uint8_t* k_codes, const uint8_t* v_codes,
                               const void* k_codebook, const void* v_codebook, const int64_t* seq_start,
                               const int32_t* seq_len, int32_t max_len, int64_t total_tokens, const void* rope_table,
                               int32_t rope_positions, float* out, void* stream) {
  if (int st = check_attn_args(d, q, k_codes, v_codes, k_codebook, v_codebook, seq_start, seq_len, max_len,
                               total_tokens, rope_table, rope_positions, out))
    return st;
  const size_t counters = static_cast<size_t>(d->batch) * d->n_kv_heads * sizeof(uint32_t);
  if (counters > kNoAllocCounterBytes)
    return fail(COMMVQ_EUNSUPPORTED, "batch x n_kv_heads = %zu exceeds the %zu arrival counters of the static scratch",
                counters / sizeof(uint32_t), kNoAllocCounterBytes / sizeof(uint32_t));
  // same partial layout as the caller-owned workspace, after the fixed counter head
  const AttnWs w = attn_ws(d, max_len);
  const size_t need = kNoAllocCounterBytes + (w.bytes - w.ml_offset);
  if (need > kNoAllocScratchBytes)
    return fail(COMMVQ_EWORKSPACE, "the call needs %zu bytes of scratch; the static scratch holds %zu", need,
                kNoAllocScratchBytes);
  void* base = nullptr;
  if (int st = hip_status(noalloc_scratch(&base, static_cast<hipStream_t>(stream)), "static scratch")) return st;
  unsigned char* ws = static_cast<unsigned char*>(base);
  unsigned char* parts = ws + kNoAllocCounterBytes;
  return launch_attn_decode(d, q, k_codes, v_codes, k_codebook, v_codebook, seq_start, seq_len, max_len,
                            total_tokens, rope_table, ws, parts, parts + (w.o_offset - w.ml_offset), out, stream);
}

size_t commvq_value_reduce_workspace_size(const commvq_dims* d, int32_t max_len) {
  if (check_dims(d) != COMMVQ_OK || max_len < 0) return 0;
  return part_bytes(d, max_len);
}

int commvq_value_reduce(const commvq_dims* d, const float* p, const uint8_t* v_codes, const void* v_codebook,
                        const int64_t* seq_start, const int32_t* seq_len, int32_t max_len, int64_t total_tokens,
                        void* workspace, size_t ws_bytes, float* out, void* stream) {
  if (int st = check_dims(d)) return st;
  if (!p || !v_codes || !v_codebook || !seq_start || !seq_len || !out)
    return fail(COMMVQ_EINVAL, "a required pointer is NULL");
  if (max_len < 0) return fail(COMMVQ_EINVAL, "max_len = %d must be >= 0", max_len);
  if (total_tokens < 0) return fail(COMMVQ_EINVAL, "total_tokens = %lld must be >= 0", (long long)total_tokens);
  if (max_len > 0 && total_tokens < 1) return fail(COMMVQ_EINVAL, "total_tokens must be >= 1 when max_len > 0");
  if (!aligned16(v_codes)) return fail(COMMVQ_EINVAL, "v_codes must be 16-byte aligned");
  const size_t need = part_bytes(d, max_len);
  if (!workspace || ws_bytes < need) return fail(COMMVQ_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  ValueReduceArgs a;
  a.p = p;
  a.p_stride = max_len;
  a.v_codes = v_codes;
  a.v_cb = v_codebook;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.total_tokens = total_tokens;
  a.n_splits = static_cast<int32_t>(n_splits_for(max_len));
  a.n_q_heads = d->n_q_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.part = static_cast<float*>(workspace);
  return hip_status(launch_value_reduce(d->dtype, packed_family(d), d->n_residuals, d->batch, a, out,
                                        static_cast<hipStream_t>(stream)),
                    "value_reduce launch");
}

int commvq_encode_greedy(const commvq_dims* d, const void* x, const void* codebook, int64_t n_tokens, uint8_t* codes,
                         int64_t total_rows, int64_t first_row, void* stream) {
  if (int st = check_dims(d)) return st;
  if (n_tokens < 0) return fail(COMMVQ_EINVAL, "n_tokens = %lld must be >= 0", (long long)n_tokens);
  if (first_row < 0 || total_rows < 0 || first_row + n_tokens > total_rows)
    return fail(COMMVQ_EINVAL, "rows [%lld, %lld) do not fit total_rows = %lld", (long long)first_row,
                (long long)(first_row + n_tokens), (long long)total_rows);
  if (n_tokens == 0) return ok();
  if (!x || !codebook || !codes) return fail(COMMVQ_EINVAL, "x, codebook and codes must be non-NULL");
  if ((n_tokens + 255) / 256 > 0x7fffffffLL) return fail(COMMVQ_EUNSUPPORTED, "n_tokens = %lld is too large",
                                                          (long long)n_tokens);
  if (packed_family(d)) {
    if (!aligned16(codes)) return fail(COMMVQ_EINVAL, "codes must be 16-byte aligned");
    return hip_status(launch_encode_greedy_bits(d->n_residuals, d->n_kv_heads, x, codebook, n_tokens,
                                                reinterpret_cast<uint32_t*>(codes), total_rows, first_row,
                                                static_cast<hipStream_t>(stream)),
                      "encode_greedy launch");
  }
  return hip_status(launch_encode_greedy(d->dtype, d->n_residuals, d->n_kv_heads, x, codebook, n_tokens, codes,
                                         total_rows, first_row, static_cast<hipStream_t>(stream)),
                    "encode_greedy launch");
}

int commvq_codebook_update(const commvq_dims* d, const void* x, const uint8_t* codes, int64_t n_tokens,
                           const void* codebook_in, void* codebook_out, void* stream) {
  if (int st = check_dims(d)) return st;
  if (n_tokens < 0) return fail(COMMVQ_EINVAL, "n_tokens = %lld must be >= 0", (long long)n_tokens);
  if (!codebook_in || !codebook_out) return fail(COMMVQ_EINVAL, "codebook_in and codebook_out must be non-NULL");
  if (n_tokens > 0 && (!x || !codes)) return fail(COMMVQ_EINVAL, "x and codes must be non-NULL");
  const bool packed = packed_family(d);
  if (packed && n_tokens > 0 && !aligned16(codes)) return fail(COMMVQ_EINVAL, "codes must be 16-byte aligned");
  // [Hkv][G][R][N][W] with G W = head_dim
  const size_t cb_bytes = static_cast<size_t>(d->n_kv_heads) * d->n_residuals * d->n_codes * kHeadDim *
                          (d->dtype == COMMVQ_F16 ? 2 : 4);
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(codebook_in), b0 = reinterpret_cast<uintptr_t>(codebook_out);
  if (a0 < b0 + cb_bytes && b0 < a0 + cb_bytes)
    return fail(COMMVQ_EINVAL, "codebook_out overlaps codebook_in (the update reads the input while writing)");
  if (packed)
    return hip_status(launch_codebook_update_bits(d->n_residuals, d->n_kv_heads, x, reinterpret_cast<const uint32_t*>(codes),
                                                  n_tokens, codebook_in, codebook_out, static_cast<hipStream_t>(stream)),
                      "codebook_update launch");
  return hip_status(launch_codebook_update(d->dtype, d->n_residuals, d->n_kv_heads, x, codes, n_tokens, codebook_in,
                                           codebook_out, static_cast<hipStream_t>(stream)),
                    "codebook_update launch");
}

int commvq_debug_unpack(const commvq_dims* d, const uint8_t* codes, int64_t total_tokens, int32_t* out, void* stream) {
  if (int st = check_dims(d)) return st;
  if (!codes || !out) return fail(COMMVQ_EINVAL, "codes and out must be non-NULL");
  if (total_tokens < 0) return fail(COMMVQ_EINVAL, "total_tokens = %lld must be >= 0", (long long)total_tokens);
  if (!aligned16(codes)) return fail(COMMVQ_EINVAL, "codes must be 16-byte aligned");
  if (packed_family(d))
    return hip_status(launch_debug_unpack_bits(d->n_residuals, d->n_kv_heads, total_tokens,
                                               reinterpret_cast<const uint32_t*>(codes), out,
                                               static_cast<hipStream_t>(stream)),
                      "debug_unpack launch");
  return hip_status(launch_debug_unpack(d->n_residuals, d->n_kv_heads, total_tokens, codes, out,
                                        static_cast<hipStream_t>(stream)),
                    "debug_unpack launch");
}

}  // extern "C"
