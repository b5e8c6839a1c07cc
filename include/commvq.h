/*
 * commvq.h: C ABI of libcommvq, decode-step attention read directly from an additive
 * vector-quantized ("CommVQ") KV cache on AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   - Each key and each value vector is quantized as a whole by additive quantization: it is the sum,
 *     group by group, of one codeword from each of R residual codebooks, so it decodes by a plain
 *     codebook product ("1-bit quantization" tag page, CommVQ abstract; "CommVQ: Commutative Vector
 *     Quantization for KV Cache Compression" summary, section Approach).
 *   - The key codebook stores, per RoPE 2-D subspace, 2x2 blocks [[a,-b],[b,a]] that commute with the
 *     RoPE rotation, so the query x codebook products are formed once per decode step and reused for
 *     every cached position; values are reduced by weighting their codes with the softmax before the
 *     codebook product (pith.science verdict for arXiv 2506.18879, pith_extraction.key_machinery and
 *     pith_extraction.forward_implications).
 *
 * Shapes and layouts (all row-major, innermost last; D = head_dim, G = n_groups, W = D / G,
 * R = n_residuals, N = n_codes, T = total cached token rows, P = D / 2 RoPE pairs):
 *   q          [B][Hq][D]          query of the new token, already rotated by the caller (dtype)
 *   k_codebook [Hkv][G][R][N][W]   key codewords; per RoPE pair u of a group the two numbers (a, b) of
 *                                  the block [[a,-b],[b,a]] (dtype)
 *   v_codebook [Hkv][G][R][N][W]   value codewords (dtype)
 *   k_codes    [Hkv][R][T][G]      uint8 code indices (N = 256: one byte per index, no packing); one
 *                                  plane per residual codebook, so a token's 16 group indices of one
 *                                  residual form one 16-byte record
 *   v_codes    [Hkv][R][T][G]      uint8
 *   seq_start  [B] int64, seq_len [B] int32: sequence b owns token rows seq_start[b] ..
 *              seq_start[b] + seq_len[b] - 1 of every KV head; its keys sit at positions 0 .. L_b - 1.
 *   out        [B][Hq][D]          fp32
 * q head h reads KV head h / (Hq / Hkv). Pair j covers dims (2j, 2j+1); RoPE frequency
 * theta_j = rope_base^(-2j/D); group g holds pairs 4g .. 4g+3 (W = 8).
 *
 * Bit-packed layout (the CommVQ pages' own code shape: one index shared by 64 dims, N = 64 codewords,
 * R up to 32 residual rounds, e.g. R = 11 for about 1 bit per scalar and R = 21 for about 2; average
 * bits R log2(N) / 64 per scalar: pith.science verdict for arXiv 2506.18879, key_machinery and the
 * referee report's minor comments; the CommVQ summary page, Limitations, names R = 11 and 21).
 * Selected by n_groups = 2, n_codes = 64:
 *   k_codebook, v_codebook [Hkv][2][R][64][64]   as above with W = 64 (group g holds pairs 32g .. 32g+31)
 *   k_codes, v_codes       [Hkv][ceil(12 R / 32)][T] little-endian uint32 words, passed through the
 *                          uint8_t pointer: token t's R x 2 six-bit indices as one bitstream, index
 *                          (r, g) at bit 6 (2 r + g) (bit k of the stream = bit k % 32 of word k / 32),
 *                          word w of token t at [kv][w][t] (one word plane per w, like the byte
 *                          layout's residual planes)
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless marked (host). Buffers are owned by the caller; the library
 *     allocates nothing, frees nothing and never synchronizes. Its only state is the static per-GPU scratch
 *     of commvq_attn_decode_noalloc.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream) and runs
 *     asynchronously. Device faults surface at the caller's next synchronization.
 *   - All argument checks run on the host before any launch; a failing call launches nothing and has
 *     no side effects. Return value: COMMVQ_OK (0) or a negative commvq_status; the thread-local
 *     commvq_last_error_detail() then names the offending argument.
 *   - Supported now: head_dim 128, Hq / Hkv = 4, and either the byte layout (n_groups 16, n_codes 256,
 *     n_residuals 1..2, dtype fp16 or fp32) or the bit-packed layout (n_groups 2, n_codes 64,
 *     n_residuals 1..32, dtype fp16), on every entry point. Other values return COMMVQ_EUNSUPPORTED.
 *   - No C++ exception crosses the ABI.
 */
#ifndef COMMVQ_H
#define COMMVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { COMMVQ_F16 = 1, COMMVQ_F32 = 2 } commvq_dtype;

typedef enum {
  COMMVQ_OK = 0,
  COMMVQ_EINVAL = -1,       /* null pointer, negative size, inconsistent shapes */
  COMMVQ_EUNSUPPORTED = -2, /* valid but not implemented (head_dim, groups, codes, residuals, GQA) */
  COMMVQ_EWORKSPACE = -3,   /* workspace (or table) smaller than the matching *_size() call asks */
  COMMVQ_EHIP = -4          /* a HIP launch failed; the detail string holds HIP's message */
} commvq_status;

typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;     /* D (128) */
  int32_t n_groups;     /* G (16, or 2 bit-packed): one code index per residual per group of W = D/G dims */
  int32_t n_residuals;  /* R (1..2, or 1..32 bit-packed): residual codebooks */
  int32_t n_codes;      /* N (256, or 64 bit-packed) */
  double rope_base;     /* RoPE base (e.g. 500000) */
  float softmax_scale;  /* e.g. 1/sqrt(D) */
  int32_t dtype;        /* commvq_dtype of q and both codebooks; outputs are fp32 */
} commvq_dims;

/* Static description of a status code. */
const char* commvq_status_string(int status);
/* Detail of the last failing call made by this thread ("" if none). */
const char* commvq_last_error_detail(void);

/* ---------------------------------------------------------------------------------------------
 * RoPE phase table: e^{i * t * theta_j} for positions t = 0 .. n_positions-1, stored as two levels in
 * three sections, each entry computed in fp64 and rounded once to fp32:
 *   fine[j][f]   = e^{i f theta_j}, f < 64, pair-major, complex fp32 (re, im)        (32 KiB)
 *   fine32g[g][h][f][p] = the same phases for pair j = 4g + 2h + p, complex fp32     (32 KiB)
 *   coarse[c][j] = e^{i 64 c theta_j}, c < ceil(n_positions / 64), complex fp32     (512 B per row)
 * The rotation of a key at position t is coarse[t >> 6][j] * fine[j][t & 63]
 * ("pith.science verdict", key_machinery: the block-diagonal rotation R_m of each 2-D sub-vector).
 * It depends only on rope_base, head_dim and the longest position, like a model's RoPE cache:
 * build it once and pass it to every commvq_attn_decode call.
 * ------------------------------------------------------------------------------------------- */
size_t commvq_rope_table_size(const commvq_dims* d /* host */, int32_t n_positions);
int commvq_rope_table(const commvq_dims* d /* host */, int32_t n_positions, void* table, size_t table_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------------------------
 * Query x key-codebook table: built once per query and shared by every cached position (pith.science verdict,
 * key_machinery; summary page, Approach):
 *   table[b][h][g][r][l][2u]   = q[b][h][2j] * a + q[b][h][2j+1] * b
 *   table[b][h][g][r][l][2u+1] = q[b][h][2j] * b - q[b][h][2j+1] * a
 * i.e. conj(q_j) * (a + i b) for pair j = (W/2) g + u and codeword (a, b) = k_codebook[kv][g][r][l][2u..2u+1]
 * (W = 8 in the byte layout, 64 in the bit-packed one).
 * Output [B][Hq][G][R][N][W] in dtype (fp16 results are rounded once from fp32).
 * k_codebook and table must be 16-byte aligned (COMMVQ_EINVAL otherwise).
 * ------------------------------------------------------------------------------------------- */
int commvq_qcodebook_table(const commvq_dims* d /* host */, const void* q, const void* k_codebook, void* table,
                           void* stream);

/* ---------------------------------------------------------------------------------------------
 * Decode-step attention over the compressed cache (pith.science verdict for arXiv 2506.18879,
 * key_machinery: keys are additive codes whose 2x2 codeword blocks commute with the RoPE rotation, so the
 * query meets the codebook once per step; forward_implications: values are weighted by the softmax before
 * the codebook product; CommVQ summary page, Approach). For every (b, h):
 *   s_t   = softmax_scale * sum_j Re( conj(q_j) * khat_{t,j} * e^{i t theta_j} ),  t < L_b
 *   khat_{t,j} = sum_r k_codebook[kv][g][r][k_codes[kv][r][seq_start[b]+t][g]][2u..2u+1]   (j = 4g+u)
 *   out[b][h] = sum_t softmax(s)_t * vhat_t,  vhat_t = sum_r v_codebook[kv][g][r][v_codes[kv][r][..][g]]
 * No key or value is dequantized to memory. Sequences with L_b = 0 produce zeros.
 * Arithmetic: codewords are read in dtype; the residual sum, the key rotation, the scores, the softmax and
 * the value accumulation run in fp32 for both dtypes (fp16 storage included), so the error does not grow
 * with the logit range. The value products round the softmax weights once: to fp16 for fp16 storage in the
 * byte layout, and, in the bit-packed layout, to the nearest multiple of 2^-19 of the split's largest weight
 * per head, binned by value index in exact integer sums. Results stay within 2e-3 (fp16 storage) and 1e-5
 * (fp32) of the exact value per output row, relative to the row's largest entry, for score spreads up to a
 * standard deviation of 12 and tokens that dominate the softmax.
 * rope_table: from commvq_rope_table with rope_positions >= max_len.
 * max_len (host) should be >= every seq_len[b], and seq_start[b] + seq_len[b] <= total_tokens (host),
 * the row count of the code arrays. The kernels cannot report a descriptor that breaks these bounds (it
 * is in device memory); they clamp it instead: start into [0, total_tokens], length into
 * [0, min(max_len, total_tokens - start)], so no read leaves the code arrays, the RoPE table or the
 * workspace. rope_table must hold at least rope_positions positions.
 * workspace: at least commvq_attn_decode_workspace_size(d, max_len) bytes, caller owned, 256-byte
 * aligned, and zero-filled before its first use: its head holds one arrival counter per (b, kv) that
 * the last workgroup of each (b, kv) resets, so every completed call leaves it zero-filled again; the
 * rest is scratch. Calls that share one workspace must not overlap in time.
 * Codes, codebooks and rope_table must be 16-byte aligned.
 * Both layouts: the bit-packed one reads its word planes [Hkv][words][T] instead of the byte planes.
 * ------------------------------------------------------------------------------------------- */
size_t commvq_attn_decode_workspace_size(const commvq_dims* d /* host */, int32_t max_len);
int commvq_attn_decode(const commvq_dims* d /* host */, const void* q, const uint8_t* k_codes, const uint8_t* v_codes,
                       const void* k_codebook, const void* v_codebook, const int64_t* seq_start,
                       const int32_t* seq_len, int32_t max_len /* host */, int64_t total_tokens /* host */,
                       const void* rope_table, int32_t rope_positions /* host */, void* workspace,
                       size_t ws_bytes /* host */, float* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * commvq_attn_decode without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments, checks,
 * kernels and result as commvq_attn_decode; the split partials and arrival counters live instead in a static
 * device array of the library, 8 MiB per GPU, which each GPU the library runs on holds from the first call
 * on that device until the process ends (that first call also clears its 64 KiB counter head with a small
 * fill kernel on `stream`). The call allocates nothing and frees nothing.
 * Limits: batch x n_kv_heads <= 16384 (COMMVQ_EUNSUPPORTED beyond) and the call's partials (per (b, q head,
 * split) 8 + 512 bytes, the commvq_attn_decode_workspace_size layout) within 8 MiB - 64 KiB
 * (COMMVQ_EWORKSPACE beyond, with the bytes needed in the detail string).
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU race (serialize them,
 * e.g. on one stream). Every completed call leaves the counters zero for the next.
 * ------------------------------------------------------------------------------------------- */
int commvq_attn_decode_noalloc(const commvq_dims* d /* host */, const void* q, const uint8_t* k_codes,
                               const uint8_t* v_codes, const void* k_codebook, const void* v_codebook,
                               const int64_t* seq_start, const int32_t* seq_len, int32_t max_len /* host */,
                               int64_t total_tokens /* host */, const void* rope_table,
                               int32_t rope_positions /* host */, float* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Value reduce with given weights, in the reordered form of the pages (pith.science verdict,
 * forward_implications: the softmax weights multiply the value codes before the codebook product):
 *   bins[g][r][l] = sum_{t < L_b} p[b][h][t] * [index (r, g) of token row seq_start[b]+t == l]
 *   out[b][h][W g + w] = sum_r sum_l bins[g][r][l] * v_codebook[kv][g][r][l][w]
 * v_codes: the byte planes [Hkv][R][T][G], or (bit-packed layout) the word planes [Hkv][words][T].
 * p: [B][Hq][max_len] fp32, any finite real values, used as given (no renormalisation); entries at
 * t >= L_b are ignored. workspace: commvq_value_reduce_workspace_size(d, max_len) bytes.
 * Resolution: the bins are integer fixed point per (b, h, work item of t): 4096 tokens for fp16 storage in the
 * byte layout, 2048 for fp32 storage and for the bit-packed layout. Each weight is rounded to a multiple of
 * 2^-B * 2^e, where 2^e is the power of two just above the item's max |p| and B = 18 (fp16 byte layout) or 19;
 * for fp32 storage its rounding residual is binned once more, at 2^-(2B+1) * 2^e. A weight below half that
 * step (about 2^-(B+1), resp. 2^-(2B+2), of the item's largest) thus contributes nothing, and every other one
 * is represented to that absolute step; the result does not depend on the order of the adds.
 * seq_start / seq_len are clamped as in commvq_attn_decode (length at most max_len and the rows left).
 * ------------------------------------------------------------------------------------------- */
size_t commvq_value_reduce_workspace_size(const commvq_dims* d /* host */, int32_t max_len);
int commvq_value_reduce(const commvq_dims* d /* host */, const float* p, const uint8_t* v_codes,
                        const void* v_codebook, const int64_t* seq_start, const int32_t* seq_len,
                        int32_t max_len /* host */, int64_t total_tokens /* host */, void* workspace,
                        size_t ws_bytes /* host */, float* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Greedy residual encoder: writes the code indices of n_tokens new keys or values into a code array
 * ("1-bit quantization" tag page, CommVQ abstract: vectors are encoded into indices of an additive
 * codebook; pith.science verdict for arXiv 2506.18879, key_machinery: R residual rounds). It stands in
 * for the pages' learned encoder, whose weights are not available: per (KV head, token, group), round
 * r = 0..R-1 picks l* = argmin_l ||res - C[kv][g][r][l]||^2 (distances in fp32; the first minimum in index
 * order) and subtracts that codeword from res (res starts as the group's W values of x).
 *   x         [Hkv][n_tokens][D] in dims->dtype, in the codebook's own frame (keys before RoPE)
 *   codebook  [Hkv][G][R][N][W] in dims->dtype
 *   codes     a [Hkv][R][total_rows][G] uint8 code array, or (bit-packed layout) word planes
 *             [Hkv][ceil(12 R / 32)][total_rows] uint32, 16-byte aligned; token t is written to row
 *             first_row + t (its whole record: one word in each plane), other rows are untouched (so new
 *             tokens can be appended to a cache in place)
 * Returns COMMVQ_EINVAL unless 0 <= first_row and first_row + n_tokens <= total_rows; n_tokens = 0 is a
 * no-op.
 * ------------------------------------------------------------------------------------------- */
int commvq_encode_greedy(const commvq_dims* d /* host */, const void* x, const void* codebook,
                         int64_t n_tokens /* host */, uint8_t* codes, int64_t total_rows /* host */,
                         int64_t first_row /* host */, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Residual codebook update: the M-step of the codebook fit (pith.science verdict for arXiv 2506.18879,
 * key_machinery: the codebook is fit by an EM-style clustering algorithm and R residual rounds refine the
 * reconstruction; "1-bit quantization" tag page, CommVQ abstract: EM training). With the E-step being an
 * assignment such as commvq_encode_greedy's, for every (kv, g, r, l):
 *   codebook_out[kv][g][r][l] = mean over tokens t whose index (r, g) is l of the round-r residual
 *                               x[kv][t][W g .. W g + W-1] - sum_{r' < r} codebook_in[kv][g][r'][index (r', g) of t]
 * (the least-squares codeword for that assignment; every round uses codebook_in for its residuals), and
 * codebook_out = codebook_in for a codeword no token selects.
 *   x             [Hkv][n_tokens][D] in dims->dtype, in the codebook's own frame (keys before RoPE)
 *   codes         [Hkv][R][n_tokens][G] uint8 (commvq_encode_greedy with first_row 0, total_rows n_tokens),
 *                 or (bit-packed layout) the word planes [Hkv][ceil(12 R / 32)][n_tokens] uint32, 16-byte
 *                 aligned
 *   codebook_in   [Hkv][G][R][N][W] in dims->dtype
 *   codebook_out  same shape and type; must not overlap codebook_in (COMMVQ_EINVAL)
 * The residuals are formed in fp64 and summed exactly (int64 fixed point), so the result does not depend on
 * the order of the adds: repeated calls give identical codebooks, each entry within one ulp of dims->dtype
 * of the exact mean.
 * n_tokens = 0 copies codebook_in (x and codes may then be NULL).
 * ------------------------------------------------------------------------------------------- */
int commvq_codebook_update(const commvq_dims* d /* host */, const void* x, const uint8_t* codes,
                           int64_t n_tokens /* host */, const void* codebook_in, void* codebook_out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Code unpack exactly as the attention kernels read codes: out[kv][r][t][g] = index (int32).
 * codes [Hkv][R][total_tokens][G] uint8, or (bit-packed layout) the word planes
 * [Hkv][ceil(12 R / 32)][total_tokens] uint32, read in the attention kernel's windows of 8 residuals (3 words).
 * Used to test the unpack bit-exactly.
 * ------------------------------------------------------------------------------------------- */
int commvq_debug_unpack(const commvq_dims* d /* host */, const uint8_t* codes, int64_t total_tokens /* host */,
                        int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COMMVQ_H */
