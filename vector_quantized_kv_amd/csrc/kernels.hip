// HIP kernels for CommVQ on gfx950 besides the fused attention kernel (attn.hip): RoPE phase table,
// query x codebook table, value reduce through code bins, and the unpack test kernel.
//
// Method sources (cited by page title and section):
//   - "1-bit quantization" tag page, CommVQ abstract: additive quantization of each KV vector, decoded by
//     a codebook product; RoPE-commutative key codebook.
//   - pith.science verdict for arXiv 2506.18879, pith_extraction.key_machinery: per 2-D subspace the key
//     codebook holds blocks that commute with the RoPE rotation, so query x codebook products are built
//     once and reused for every cached position; pith_extraction.forward_implications: the softmax
//     weights multiply the value codes before the codebook product.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"

namespace commvq {

typedef _Float16 f16;

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return static_cast<float>(*p);
}

// ------------------------------------------------------------------------------------ RoPE table
// One thread per entry, over three sections: fine fp32 pair-major (entry j * 64 + f = e^{i f theta_j}),
// fine packed fp16 group-major (entry (g * 64 + f) * 4 + u for pair j = 4g + u, (cos, sin) rounded once
// from fp64), coarse fp32 position-major (entry c * 64 + j = e^{i 64 c theta_j}).
__global__ void rope_table_kernel(double base, int64_t n_coarse, float2* out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  constexpr int64_t kFine = static_cast<int64_t>(kFineRows) * kPairs;
  if (idx >= 2 * kFine + n_coarse * kPairs) return;
  int j;
  double pos;
  if (idx < kFine) {
    j = static_cast<int>(idx / kFineRows);
    pos = static_cast<double>(idx % kFineRows);
  } else if (idx < 2 * kFine) {
    const int k = static_cast<int>(idx - kFine);
    j = 4 * (k >> 8) + (k & 3);
    pos = static_cast<double>((k >> 2) & 63);
  } else {
    j = static_cast<int>((idx - 2 * kFine) % kPairs);
    pos = 64.0 * static_cast<double>((idx - 2 * kFine) / kPairs);
  }
  const double theta = pow(base, -2.0 * j / static_cast<double>(kHeadDim));
  double s, c;
  sincos(pos * theta, &s, &c);
  if (idx < kFine) {
    out[idx] = make_float2(static_cast<float>(c), static_cast<float>(s));
  } else if (idx < 2 * kFine) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    reinterpret_cast<h2*>(out + kRopeFine16Offset)[idx - kFine] = (h2){static_cast<f16>(c), static_cast<f16>(s)};
  } else {
    out[kRopeCoarseOffset + (idx - 2 * kFine)] = make_float2(static_cast<float>(c), static_cast<float>(s));
  }
}

hipError_t launch_rope_table(double base, int32_t n_positions, float2* table, hipStream_t s) {
  const int64_t n_coarse = rope_coarse_rows(n_positions);
  const int64_t n = 2LL * kFineRows * kPairs + n_coarse * kPairs;
  rope_table_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(base, n_coarse, table);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- query x codebook table
// grid (G*R, Hq, B), block N: thread l writes the W/2 complex entries of code l. Byte layout G = 16, N = 256,
// W = 8; bit-packed layout G = 2, N = 64, W = 64.
template <typename T, int G, int N>
__global__ void __launch_bounds__(256) qtable_kernel(const T* q, const T* kcb, T* out, int Hq, int Hkv, int R) {
  constexpr int W = kHeadDim / G;
  const int gr = blockIdx.x, h = blockIdx.y, b = blockIdx.z, l = threadIdx.x;
  const int g = gr / R, r = gr % R, kv = h / (Hq / Hkv);
  const T* qq = q + (static_cast<int64_t>(b) * Hq + h) * kHeadDim + W * g;
  const T* c = kcb + (((static_cast<int64_t>(kv) * G + g) * R + r) * N + l) * W;
  T* o = out + ((((static_cast<int64_t>(b) * Hq + h) * G + g) * R + r) * N + l) * W;
#pragma unroll
  for (int u = 0; u < W / 2; ++u) {
    const float q0 = ld(qq + 2 * u), q1 = ld(qq + 2 * u + 1), a = ld(c + 2 * u), bb = ld(c + 2 * u + 1);
    o[2 * u] = static_cast<T>(q0 * a + q1 * bb);
    o[2 * u + 1] = static_cast<T>(q0 * bb - q1 * a);
  }
}

hipError_t launch_qtable(int dtype, bool packed, int R, int B, int Hq, int Hkv, const void* q, const void* kcb,
                         void* out, hipStream_t s) {
  if (packed) {  // fp16 only
    qtable_kernel<f16, kWideGroups, kWideCodes><<<dim3(kWideGroups * R, Hq, B), kWideCodes, 0, s>>>(
        static_cast<const f16*>(q), static_cast<const f16*>(kcb), static_cast<f16*>(out), Hq, Hkv, R);
    return hipGetLastError();
  }
  dim3 grid(kGroups * R, Hq, B);
  if (dtype == COMMVQ_F16)
    qtable_kernel<f16, kGroups, kCodes><<<grid, kCodes, 0, s>>>(static_cast<const f16*>(q),
                                                                static_cast<const f16*>(kcb), static_cast<f16*>(out),
                                                                Hq, Hkv, R);
  else
    qtable_kernel<float, kGroups, kCodes><<<grid, kCodes, 0, s>>>(static_cast<const float*>(q),
                                                                  static_cast<const float*>(kcb),
                                                                  static_cast<float*>(out), Hq, Hkv, R);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------- value bins
// Fixed-point bins: LDS float atomics are slow on this chip, integer ones are not; weights are
// scaled by `fx_scale` (so |w * fx_scale| <= 2^20) and rounded, which keeps a 1024-token split's bin
// sums inside int32. bins layout [kGqa][kGroups][R][kCodes].
template <int R, int TPT>
__device__ __forceinline__ void bin_weights(int32_t* bins, const uint4 (&vc)[TPT][R], const float (&w)[TPT][kGqa],
                                            const bool (&valid)[TPT], const float (&fx_scale)[kGqa]) {
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    if (!valid[k]) continue;
    int32_t fx[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) fx[h] = static_cast<int32_t>(rintf(w[k][h] * fx_scale[h]));
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t l = code_index(vc[k][r], g);
#pragma unroll
        for (int h = 0; h < kGqa; ++h) atomicAdd(&bins[((h * kGroups + g) * R + r) * kCodes + l], fx[h]);
      }
  }
}

// o[h][8g+w] = sum_r sum_l bins[h][g][r][l] * CV[g][r][l][w] / fx_scale[h]; thread handles 2 outputs.
template <typename T, int R>
__device__ __forceinline__ void contract_bins(const int32_t* bins, const T* vcb, const float (&fx_scale)[kGqa],
                                              float* part_base /* [kGqa] rows of kPartFloats */,
                                              int64_t part_row_stride) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i, h = idx >> 7, d = idx & 127, g = d >> 3, w = d & 7;
    float acc = 0.f;
    for (int r = 0; r < R; ++r) {
      const int32_t* bb = bins + ((h * kGroups + g) * R + r) * kCodes;
      const T* cv = vcb + ((static_cast<int64_t>(g) * R + r) * kCodes) * kGroupDim + w;
      for (int l = 0; l < kCodes; ++l) acc = fmaf(static_cast<float>(bb[l]), ld(cv + l * kGroupDim), acc);
    }
    part_base[h * part_row_stride + 4 + d] = acc / fx_scale[h];
  }
}

// ----------------------------------------------------------------------------------- value reduce
// The reordered value reduce of the pages: weights are binned by value code (bin_weights), then the
// bins are contracted with the value codebook (contract_bins). One workgroup per (sequence, KV head,
// 1024-token split); partial outputs are summed by combine_sum_kernel. Fixed-point scale per head is
// 2^20 / max|p| over the split, so any finite weights bin exactly up to that relative resolution.
template <typename T, int R>
__global__ void __launch_bounds__(256) value_reduce_kernel(const ValueReduceArgs a) {
  constexpr int TPT = kSplitTokens / 256;
  __shared__ float red[4][kGqa];
  __shared__ __attribute__((aligned(16))) int32_t work[kGqa * kGroups * R * kCodes];
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.p_stride, a.total_tokens);
  const int L = sb.len;
  const int t0 = split * kSplitTokens;
  if (t0 >= L) return;
  const int64_t row0 = sb.start + t0;
  const int h0 = kv * kGqa;
  const int wave = tid >> 6, lane = tid & 63;
  bool valid[TPT];
  float w[TPT][kGqa];
  uint4 vc[TPT][R];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = t0 + tid + 256 * k;
    valid[k] = t < L;
#pragma unroll
    for (int h = 0; h < kGqa; ++h)
      w[k][h] = valid[k] ? a.p[(static_cast<int64_t>(b) * a.n_q_heads + h0 + h) * a.p_stride + t] : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
      vc[k][r] = valid[k] ? load_code_record(a.v_codes, a.total_tokens, kv, row0 + tid + 256 * k, R, r)
                          : make_uint4(0, 0, 0, 0);
  }
  for (int i = tid; i < kGqa * kGroups * R * kCodes; i += 256) work[i] = 0;
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < TPT; ++k) mx = fmaxf(mx, fabsf(w[k][h]));
    mx = wave_max(mx);
    if (lane == 0) red[wave][h] = mx;
  }
  __syncthreads();
  float fx_scale[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    const float mx = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
    fx_scale[h] = mx > 0.f ? 1048576.f / mx : 1.f;
  }
  bin_weights<R, TPT>(work, vc, w, valid, fx_scale);
  __syncthreads();
  float* part = a.part + ((static_cast<int64_t>(b) * a.n_q_heads + h0) * a.n_splits + split) * kPartFloats;
  const int64_t row_stride = static_cast<int64_t>(a.n_splits) * kPartFloats;
  const T* vcb = static_cast<const T*>(a.v_cb) + static_cast<int64_t>(kv) * kGroups * R * kCodes * kGroupDim;
  contract_bins<T, R>(work, vcb, fx_scale, part, row_stride);
}

__global__ void __launch_bounds__(128) combine_sum_kernel(const float* part, const ValueReduceArgs a, float* out) {
  const int bh = blockIdx.x, b = bh / a.n_q_heads, d = threadIdx.x;
  const int L = seq_bounds(a.seq_start, a.seq_len, b, a.p_stride, a.total_tokens).len;  // as value_reduce_kernel
  const int n_splits = a.n_splits;
  const int ns = (L + kSplitTokens - 1) / kSplitTokens;
  const float* p = part + static_cast<int64_t>(bh) * n_splits * kPartFloats;
  float acc = 0.f;
  for (int s = 0; s < ns; ++s) acc += p[s * kPartFloats + 4 + d];
  out[static_cast<int64_t>(bh) * kHeadDim + d] = acc;
}

// Bit-packed records (G = 2, N = 64, W = 64, R up to 32): the same split, fixed-point bins and partials.
// Bins [kGqa][2][R][64] (64 KiB at R = 32); each token reads its R x 2 indices field by field.
__global__ void __launch_bounds__(256) value_reduce_bits_kernel(const ValueReduceArgs a, int R) {
  constexpr int TPT = kSplitTokens / 256;
  constexpr int G = kWideGroups, N = kWideCodes, W = kHeadDim / G;
  __shared__ float red[4][kGqa];
  __shared__ __attribute__((aligned(16))) int32_t bins[kGqa * G * kWideMaxResiduals * N];
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.p_stride, a.total_tokens);
  const int L = sb.len;
  const int t0 = split * kSplitTokens;
  if (t0 >= L) return;
  const int64_t row0 = sb.start + t0;
  const int h0 = kv * kGqa;
  const int wave = tid >> 6, lane = tid & 63;
  const int Wd = wide_record_words(R);
  const uint32_t* words = reinterpret_cast<const uint32_t*>(a.v_codes);
  bool valid[TPT];
  float w[TPT][kGqa];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = t0 + tid + 256 * k;
    valid[k] = t < L;
#pragma unroll
    for (int h = 0; h < kGqa; ++h)
      w[k][h] = valid[k] ? a.p[(static_cast<int64_t>(b) * a.n_q_heads + h0 + h) * a.p_stride + t] : 0.f;
  }
  for (int i = tid; i < kGqa * G * R * N; i += 256) bins[i] = 0;
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < TPT; ++k) mx = fmaxf(mx, fabsf(w[k][h]));
    mx = wave_max(mx);
    if (lane == 0) red[wave][h] = mx;
  }
  __syncthreads();
  float fx_scale[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    const float mx = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
    fx_scale[h] = mx > 0.f ? 1048576.f / mx : 1.f;
  }
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    if (!valid[k]) continue;
    int32_t fx[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) fx[h] = static_cast<int32_t>(rintf(w[k][h] * fx_scale[h]));
    const uint32_t* rec = words + (static_cast<int64_t>(kv) * a.total_tokens + row0 + tid + 256 * k) * Wd;
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t l = packed_field(rec, r, g);
#pragma unroll
        for (int h = 0; h < kGqa; ++h) atomicAdd(&bins[((h * G + g) * R + r) * N + l], fx[h]);
      }
  }
  __syncthreads();
  // o[h][64g + w] = sum_r sum_l bins[h][g][r][l] * CV[g][r][l][w] / fx_scale[h]; each thread 2 outputs
  float* part = a.part + ((static_cast<int64_t>(b) * a.n_q_heads + h0) * a.n_splits + split) * kPartFloats;
  const int64_t row_stride = static_cast<int64_t>(a.n_splits) * kPartFloats;
  const f16* vcb = static_cast<const f16*>(a.v_cb) + static_cast<int64_t>(kv) * G * R * N * W;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i, h = idx >> 7, d = idx & 127, g = d / W, wd = d % W;
    float acc = 0.f;
    for (int r = 0; r < R; ++r) {
      const int32_t* bb = bins + ((h * G + g) * R + r) * N;
      const f16* cv = vcb + (static_cast<int64_t>(g) * R + r) * N * W + wd;
      for (int l = 0; l < N; ++l) acc = fmaf(static_cast<float>(bb[l]), static_cast<float>(cv[l * W]), acc);
    }
    part[h * row_stride + 4 + d] = acc / fx_scale[h];
  }
}

hipError_t launch_value_reduce(int dtype, bool packed, int R, int B, const ValueReduceArgs& a, float* out,
                               hipStream_t s) {
  dim3 grid(a.n_splits, a.n_kv_heads, B);
  if (packed) {  // fp16 only
    value_reduce_bits_kernel<<<grid, 256, 0, s>>>(a, R);
  } else if (dtype == COMMVQ_F16) {
    if (R == 1) value_reduce_kernel<f16, 1><<<grid, 256, 0, s>>>(a);
    else value_reduce_kernel<f16, 2><<<grid, 256, 0, s>>>(a);
  } else {
    if (R == 1) value_reduce_kernel<float, 1><<<grid, 256, 0, s>>>(a);
    else value_reduce_kernel<float, 2><<<grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_sum_kernel<<<dim3(B * a.n_q_heads), dim3(128), 0, s>>>(a.part, a, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------- unpack test
// One thread per (kv, row, residual): the 16-byte record goes through code_index like every kernel.
__global__ void debug_unpack_kernel(const uint8_t* codes, int64_t total_tokens, int R, int64_t n_records,
                                    int32_t* out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n_records) return;
  const uint4 w = *reinterpret_cast<const uint4*>(codes + idx * 16);
#pragma unroll
  for (int g = 0; g < kGroups; ++g) out[idx * kGroups + g] = static_cast<int32_t>(code_index(w, g));
}

hipError_t launch_debug_unpack(int R, int Hkv, int64_t total_tokens, const uint8_t* codes, int32_t* out,
                               hipStream_t s) {
  const int64_t n = static_cast<int64_t>(Hkv) * total_tokens * R;
  if (n == 0) return hipSuccess;
  debug_unpack_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(codes, total_tokens, R, n,
                                                                                      out);
  return hipGetLastError();
}

// Bit-packed records: one thread per (kv, token, window c); it reads the window's two words and unpacks
// them with the same window functions the attention kernel uses. out is [Hkv][R][T][2] int32.
__global__ void debug_unpack_bits_kernel(const uint32_t* words, int64_t total_tokens, int R, int Wd, int n_windows,
                                         int64_t n_items, int32_t* out) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= n_items) return;
  const int c = static_cast<int>(item % n_windows);
  const int64_t kt = item / n_windows;  // kv * T + t
  const int64_t kv = kt / total_tokens, t = kt % total_tokens;
  const uint32_t* rec = words + kt * Wd;
  const int w0 = packed_window_word(c);
  uint32_t x0, x1;
  packed_window(rec[w0], rec[min(w0 + 1, Wd - 1)], packed_window_shift(c), x0, x1);
  uint32_t idx[2 * kWideResPerPass];
  idx[0] = packed_index<0>(x0, x1);
  idx[1] = packed_index<1>(x0, x1);
  idx[2] = packed_index<2>(x0, x1);
  idx[3] = packed_index<3>(x0, x1);
  idx[4] = packed_index<4>(x0, x1);
  idx[5] = packed_index<5>(x0, x1);
  idx[6] = packed_index<6>(x0, x1);
  idx[7] = packed_index<7>(x0, x1);
  static_assert(kWideResPerPass == 4, "eight indices per window");
#pragma unroll
  for (int rho = 0; rho < kWideResPerPass; ++rho) {
    const int r = kWideResPerPass * c + rho;
    if (r >= R) break;
#pragma unroll
    for (int g = 0; g < kWideGroups; ++g)
      out[((kv * R + r) * total_tokens + t) * kWideGroups + g] = static_cast<int32_t>(idx[2 * rho + g]);
  }
}

hipError_t launch_debug_unpack_bits(int R, int Hkv, int64_t total_tokens, const uint32_t* words, int32_t* out,
                                    hipStream_t s) {
  const int n_windows = (R + kWideResPerPass - 1) / kWideResPerPass;
  const int64_t n = static_cast<int64_t>(Hkv) * total_tokens * n_windows;
  if (n == 0) return hipSuccess;
  debug_unpack_bits_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(
      words, total_tokens, R, wide_record_words(R), n_windows, n, out);
  return hipGetLastError();
}

// ----------------------------------------------------------------------- greedy residual encoder
// Writes the code indices of new tokens ("1-bit quantization" tag page, CommVQ abstract: keys and values
// are encoded into indices of an additive codebook; pith.science verdict for arXiv 2506.18879,
// key_machinery: R residual rounds refine the reconstruction). Greedy stand-in for the pages' learned
// encoder: per (token, group), round r picks l* = argmin_l ||res - C[g][r][l]||^2 in fp32 (the first
// minimum in index order) and subtracts C[g][r][l*].
// One thread per (token, group); a workgroup covers 256 tokens of one (KV head, group), whose R x 256
// codewords sit in LDS as fp32, so all lanes of a wave read the same codeword (an LDS broadcast).
template <typename T, int R>
__global__ void __launch_bounds__(256) encode_greedy_kernel(const T* x, const T* cb, int64_t n, uint8_t* codes,
                                                            int64_t total_rows, int64_t first_row) {
  const int g = blockIdx.y, kv = blockIdx.z;
  __shared__ float4 cw[R * kCodes * 2];
  const T* cbg = cb + (static_cast<int64_t>(kv) * kGroups + g) * R * kCodes * kGroupDim;
  for (int i = threadIdx.x; i < R * kCodes; i += blockDim.x) {  // i = r * 256 + l
    const T* c = cbg + static_cast<int64_t>(i) * kGroupDim;
    cw[2 * i] = make_float4(ld(c), ld(c + 1), ld(c + 2), ld(c + 3));
    cw[2 * i + 1] = make_float4(ld(c + 4), ld(c + 5), ld(c + 6), ld(c + 7));
  }
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const T* xv = x + (static_cast<int64_t>(kv) * n + t) * kHeadDim + g * kGroupDim;
  float res[kGroupDim];
#pragma unroll
  for (int w = 0; w < kGroupDim; ++w) res[w] = ld(xv + w);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float best = INFINITY;
    int bl = 0;
    for (int l = 0; l < kCodes; ++l) {
      const float4 c0 = cw[2 * (r * kCodes + l)], c1 = cw[2 * (r * kCodes + l) + 1];
      const float c[kGroupDim] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      float dd = 0.f;
#pragma unroll
      for (int w = 0; w < kGroupDim; ++w) {
        const float e = res[w] - c[w];
        dd = fmaf(e, e, dd);
      }
      if (dd < best) {  // strict: ties keep the lowest index
        best = dd;
        bl = l;
      }
    }
    codes[((static_cast<int64_t>(kv) * R + r) * total_rows + first_row + t) * kGroups + g] = static_cast<uint8_t>(bl);
    const float4 c0 = cw[2 * (r * kCodes + bl)], c1 = cw[2 * (r * kCodes + bl) + 1];
    const float c[kGroupDim] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int w = 0; w < kGroupDim; ++w) res[w] -= c[w];
  }
}

// ------------------------------------------------------------------------ residual codebook M-step
// One workgroup per (group g, round r, KV head): every token adds its round-r residual (x_g minus the input
// codewords its earlier rounds select) to the bin of its round-r index; then thread l writes codeword l as
// the bin mean, or the input codeword when no token selects it. As in the bit-packed M-step below, the
// residual is kept in fp64 and the bins are int64 fixed point (integer LDS atomics; the scale 2^62 / (bound n)
// with bound = max|x_g| + r max|earlier codeword| keeps every sum inside int64), so the sums are exact and
// the result does not depend on the order of the adds.
template <typename T, int R>
__global__ void __launch_bounds__(256) codebook_update_kernel(const T* x, const uint8_t* codes, int64_t n,
                                                              const T* cb_in, T* cb_out) {
  const int g = blockIdx.x, r = blockIdx.y, kv = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ unsigned long long sum[kCodes * kGroupDim];
  __shared__ uint32_t cnt[kCodes];
  __shared__ float red[2][4];
  for (int i = tid; i < kCodes * kGroupDim; i += blockDim.x) sum[i] = 0ull;
  for (int i = tid; i < kCodes; i += blockDim.x) cnt[i] = 0u;
  const T* cbg = cb_in + (static_cast<int64_t>(kv) * kGroups + g) * R * kCodes * kGroupDim;  // [R][N][W]
  float xmax = 0.f, cmax = 0.f;
  for (int i = tid; i < r * kCodes * kGroupDim; i += blockDim.x) cmax = fmaxf(cmax, fabsf(ld(cbg + i)));
  for (int64_t t = tid; t < n; t += blockDim.x) {
    const T* xv = x + (static_cast<int64_t>(kv) * n + t) * kHeadDim + g * kGroupDim;
#pragma unroll
    for (int w = 0; w < kGroupDim; ++w) xmax = fmaxf(xmax, fabsf(ld(xv + w)));
  }
  xmax = wave_max(xmax);
  cmax = wave_max(cmax);
  if (lane == 0) {
    red[0][wave] = xmax;
    red[1][wave] = cmax;
  }
  __syncthreads();
  const double bound = static_cast<double>(fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]))) +
                       r * static_cast<double>(fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3])));
  const double scale = bound > 0.0 && n > 0 ? ldexp(1.0, 62) / (bound * static_cast<double>(n)) : 1.0;
  for (int64_t t = tid; t < n; t += blockDim.x) {
    const T* xv = x + (static_cast<int64_t>(kv) * n + t) * kHeadDim + g * kGroupDim;
    double res[kGroupDim];
#pragma unroll
    for (int w = 0; w < kGroupDim; ++w) res[w] = static_cast<double>(ld(xv + w));
    for (int rp = 0; rp < r; ++rp) {
      const int l = codes[((static_cast<int64_t>(kv) * R + rp) * n + t) * kGroups + g];
      const T* c = cbg + (static_cast<int64_t>(rp) * kCodes + l) * kGroupDim;
#pragma unroll
      for (int w = 0; w < kGroupDim; ++w) res[w] -= static_cast<double>(ld(c + w));
    }
    const int l = codes[((static_cast<int64_t>(kv) * R + r) * n + t) * kGroups + g];
#pragma unroll
    for (int w = 0; w < kGroupDim; ++w)
      atomicAdd(&sum[l * kGroupDim + w], static_cast<unsigned long long>(static_cast<long long>(rint(res[w] * scale))));
    atomicAdd(&cnt[l], 1u);
  }
  __syncthreads();
  for (int l = tid; l < kCodes; l += blockDim.x) {
    const int64_t o = ((static_cast<int64_t>(kv) * kGroups + g) * R + r) * kCodes * kGroupDim + l * kGroupDim;
    const uint32_t c = cnt[l];
#pragma unroll
    for (int w = 0; w < kGroupDim; ++w)
      cb_out[o + w] = c > 0 ? static_cast<T>(static_cast<double>(static_cast<long long>(sum[l * kGroupDim + w])) /
                                             (scale * c))
                            : cb_in[o + w];
  }
}

hipError_t launch_codebook_update(int dtype, int R, int Hkv, const void* x, const uint8_t* codes, int64_t n,
                                  const void* cb_in, void* cb_out, hipStream_t s) {
  const dim3 grid(kGroups, R, Hkv);
  if (dtype == COMMVQ_F16) {
    if (R == 1)
      codebook_update_kernel<f16, 1><<<grid, 256, 0, s>>>(static_cast<const f16*>(x), codes, n,
                                                          static_cast<const f16*>(cb_in), static_cast<f16*>(cb_out));
    else
      codebook_update_kernel<f16, 2><<<grid, 256, 0, s>>>(static_cast<const f16*>(x), codes, n,
                                                          static_cast<const f16*>(cb_in), static_cast<f16*>(cb_out));
  } else {
    if (R == 1)
      codebook_update_kernel<float, 1><<<grid, 256, 0, s>>>(static_cast<const float*>(x), codes, n,
                                                            static_cast<const float*>(cb_in),
                                                            static_cast<float*>(cb_out));
    else
      codebook_update_kernel<float, 2><<<grid, 256, 0, s>>>(static_cast<const float*>(x), codes, n,
                                                            static_cast<const float*>(cb_in),
                                                            static_cast<float*>(cb_out));
  }
  return hipGetLastError();
}

// Bit-packed records (one index per 64 dims: G = 2, N = 64, R up to 32): the same greedy residual rounds.
// One thread per token and one group at a time (a 64-dim fp32 residual in registers). A workgroup's 256
// tokens take the rounds together: round r's codebook of the group (64 codewords x 64 dims, 16 KiB) sits in
// LDS as fp32, and all lanes read the same codeword (a broadcast). The first minimum of the fp32 squared
// distance is chosen and subtracted. Index (r, g) goes to bit 12 r + 6 g of the token's record: group 0's
// pass stores every word, group 1's pass ORs its fields into them (ceil(12 R / 32) words per token).
__global__ void __launch_bounds__(256) encode_greedy_bits_kernel(const f16* x, const f16* cb, int R, int64_t n,
                                                                 uint32_t* words, int64_t total_rows,
                                                                 int64_t first_row) {
  constexpr int W = kHeadDim / kWideGroups, N = kWideCodes;
  constexpr int kTabF4 = N * W / 4;  // float4 entries per (group, round) codebook
  __shared__ float4 cw[kTabF4];
  const int kv = blockIdx.y;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool live = t < n;
  const int64_t tt = live ? t : n - 1;  // clamped: every thread takes part in the rounds (and their barriers)
  const int Wd = wide_record_words(R);
  uint32_t* rec = words + (static_cast<int64_t>(kv) * total_rows + first_row + tt) * Wd;
  for (int g = 0; g < kWideGroups; ++g) {
    float res[W];
    const f16* xv = x + (static_cast<int64_t>(kv) * n + tt) * kHeadDim + g * W;
#pragma unroll
    for (int w = 0; w < W; ++w) res[w] = static_cast<float>(xv[w]);
    uint64_t acc = 0;  // acc bit 0 = record bit 32 * word
    int word = 0;
    auto flush = [&]() {
      uint32_t v = static_cast<uint32_t>(acc);
      if (live) {
        if (g > 0) v |= rec[word];
        rec[word] = v;
      }
      acc >>= 32;
      ++word;
    };
    for (int r = 0; r < R; ++r) {
      __syncthreads();  // every thread is done with the previous round's codewords
      for (int i = threadIdx.x; i < kTabF4; i += blockDim.x) {
        const f16* c = cb + ((static_cast<int64_t>(kv) * kWideGroups + g) * R + r) * N * W + i * 4;
        cw[i] = make_float4(static_cast<float>(c[0]), static_cast<float>(c[1]), static_cast<float>(c[2]),
                            static_cast<float>(c[3]));
      }
      __syncthreads();
      float best = INFINITY;
      int bi = 0;
      for (int l = 0; l < N; ++l) {
        const float4* c = cw + l * (W / 4);
        float dsum = 0.f;
#pragma unroll
        for (int q = 0; q < W / 4; ++q) {
          const float4 v = c[q];
          const float e0 = res[4 * q] - v.x, e1 = res[4 * q + 1] - v.y;
          const float e2 = res[4 * q + 2] - v.z, e3 = res[4 * q + 3] - v.w;
          dsum = fmaf(e0, e0, dsum);
          dsum = fmaf(e1, e1, dsum);
          dsum = fmaf(e2, e2, dsum);
          dsum = fmaf(e3, e3, dsum);
        }
        if (dsum < best) {  // strict: ties keep the lowest index
          best = dsum;
          bi = l;
        }
      }
      const float4* c = cw + bi * (W / 4);
#pragma unroll
      for (int q = 0; q < W / 4; ++q) {
        const float4 v = c[q];
        res[4 * q] -= v.x;
        res[4 * q + 1] -= v.y;
        res[4 * q + 2] -= v.z;
        res[4 * q + 3] -= v.w;
      }
      acc |= static_cast<uint64_t>(bi) << (kWideBits * (kWideGroups * r + g) - 32 * word);
      // the group's next field starts at or past bit 32 of acc: the low word is final for this group
      if (kWideBits * (kWideGroups * (r + 1) + g) - 32 * word >= 32) flush();
    }
    while (word < Wd) flush();
  }
}

// Residual codebook M-step on bit-packed records. One workgroup per (group g, slice of kUpdSlice dims, KV
// head): every round's bins for the slice ([R][64][kUpdSlice]), their counts and the slice of every input
// codeword (fp32) sit in LDS. Each token walks its rounds once: it adds its residual slice to bin (r, l),
// then subtracts the input codeword's slice, so round r's bins receive x_g - sum_{r' < r} C_in[g][r'][l_r'].
// The residual is kept in fp64, where x and the fp16 codewords, and their sums over the rounds, are exact, so
// late rounds carry no accumulated rounding. The bins are int64 fixed point (LDS float atomics are slow on
// this chip, integer ones are not): a first pass bounds every residual by max|x slice| + R max|codeword
// slice|, and the scale 2^62 / (bound n) keeps each term within 2^62 / n, so no bin can overflow. The sums
// are exact, so the result does not depend on the order of the adds; only the final fp16 rounding remains.
// Thread i then writes entry i of the slice as the bin mean, or the input value when no token selects the
// codeword.
constexpr int kUpdSlice = 4;
__global__ void __launch_bounds__(256) codebook_update_bits_kernel(const f16* x, const uint32_t* words, int R,
                                                                   int64_t n, const f16* cb_in, f16* cb_out) {
  constexpr int G = kWideGroups, N = kWideCodes, W = kHeadDim / G, kSlices = W / kUpdSlice;
  static_assert(kUpdSlice == 4, "one float4 of codeword slice per (round, code)");
  __shared__ unsigned long long sum[kWideMaxResiduals * N * kUpdSlice];
  __shared__ float4 cws[kWideMaxResiduals * N];
  __shared__ uint32_t cnt[kWideMaxResiduals * N];
  __shared__ float red[2][4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = blockIdx.x / kSlices, s = blockIdx.x % kSlices, kv = blockIdx.y;
  const int64_t cb_base = (static_cast<int64_t>(kv) * G + g) * R * N * W + s * kUpdSlice;  // + (r N + l) W + w
  for (int i = tid; i < R * N * kUpdSlice; i += blockDim.x) sum[i] = 0ull;
  float cmax = 0.f, xmax = 0.f;
  for (int i = tid; i < R * N; i += blockDim.x) {
    const f16* c = cb_in + cb_base + static_cast<int64_t>(i) * W;
    const float4 v = make_float4(static_cast<float>(c[0]), static_cast<float>(c[1]), static_cast<float>(c[2]),
                                 static_cast<float>(c[3]));
    cws[i] = v;
    cnt[i] = 0u;
    cmax = fmaxf(cmax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  for (int64_t t = tid; t < n; t += blockDim.x) {
    const f16* xv = x + (static_cast<int64_t>(kv) * n + t) * kHeadDim + g * W + s * kUpdSlice;
#pragma unroll
    for (int w = 0; w < kUpdSlice; ++w) xmax = fmaxf(xmax, fabsf(static_cast<float>(xv[w])));
  }
  xmax = wave_max(xmax);
  cmax = wave_max(cmax);
  if (lane == 0) {
    red[0][wave] = xmax;
    red[1][wave] = cmax;
  }
  __syncthreads();
  const float bound = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3])) +
                      static_cast<float>(R) * fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  const double scale = bound > 0.f && n > 0 ? ldexp(1.0, 62) / (static_cast<double>(bound) * static_cast<double>(n))
                                            : 1.0;
  const int Wd = wide_record_words(R);
  for (int64_t t = tid; t < n; t += blockDim.x) {
    const uint32_t* rec = words + (static_cast<int64_t>(kv) * n + t) * Wd;
    const f16* xv = x + (static_cast<int64_t>(kv) * n + t) * kHeadDim + g * W + s * kUpdSlice;
    double res[kUpdSlice];
#pragma unroll
    for (int w = 0; w < kUpdSlice; ++w) res[w] = static_cast<double>(static_cast<float>(xv[w]));
    for (int r = 0; r < R; ++r) {
      const int l = static_cast<int>(packed_field(rec, r, g));
      // the codeword read goes out before the atomics: LDS operations complete in order, so waiting for it
      // afterwards would also wait for every atomic of the round
      const float4 c = cws[r * N + l];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int w = 0; w < kUpdSlice; ++w)
        atomicAdd(&sum[(r * N + l) * kUpdSlice + w],
                  static_cast<unsigned long long>(static_cast<long long>(rint(res[w] * scale))));
      atomicAdd(&cnt[r * N + l], 1u);
      res[0] -= c.x;
      res[1] -= c.y;
      res[2] -= c.z;
      res[3] -= c.w;
    }
  }
  __syncthreads();
  for (int i = tid; i < R * N * kUpdSlice; i += blockDim.x) {
    const int rl = i / kUpdSlice, w = i % kUpdSlice;  // rl = r N + l
    const int64_t o = cb_base + static_cast<int64_t>(rl) * W + w;
    const uint32_t c = cnt[rl];
    const double mean = static_cast<double>(static_cast<long long>(sum[i])) / (scale * c);
    cb_out[o] = c > 0 ? static_cast<f16>(static_cast<float>(mean)) : cb_in[o];
  }
}

hipError_t launch_codebook_update_bits(int R, int Hkv, const void* x, const uint32_t* words, int64_t n,
                                       const void* cb_in, void* cb_out, hipStream_t s) {
  const dim3 grid(kWideGroups * (kHeadDim / kWideGroups / kUpdSlice), Hkv);
  codebook_update_bits_kernel<<<grid, 256, 0, s>>>(static_cast<const f16*>(x), words, R, n,
                                                   static_cast<const f16*>(cb_in), static_cast<f16*>(cb_out));
  return hipGetLastError();
}

hipError_t launch_encode_greedy_bits(int R, int Hkv, const void* x, const void* cb, int64_t n, uint32_t* words,
                                     int64_t total_rows, int64_t first_row, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256), Hkv);
  encode_greedy_bits_kernel<<<grid, 256, 0, s>>>(static_cast<const f16*>(x), static_cast<const f16*>(cb), R, n, words,
                                                 total_rows, first_row);
  return hipGetLastError();
}

hipError_t launch_encode_greedy(int dtype, int R, int Hkv, const void* x, const void* cb, int64_t n, uint8_t* codes,
                                int64_t total_rows, int64_t first_row, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256), kGroups, Hkv);
  if (dtype == COMMVQ_F16) {
    if (R == 1)
      encode_greedy_kernel<f16, 1><<<grid, 256, 0, s>>>(static_cast<const f16*>(x), static_cast<const f16*>(cb), n,
                                                         codes, total_rows, first_row);
    else
      encode_greedy_kernel<f16, 2><<<grid, 256, 0, s>>>(static_cast<const f16*>(x), static_cast<const f16*>(cb), n,
                                                         codes, total_rows, first_row);
  } else {
    if (R == 1)
      encode_greedy_kernel<float, 1><<<grid, 256, 0, s>>>(static_cast<const float*>(x), static_cast<const float*>(cb),
                                                           n, codes, total_rows, first_row);
    else
      encode_greedy_kernel<float, 2><<<grid, 256, 0, s>>>(static_cast<const float*>(x), static_cast<const float*>(cb),
                                                           n, codes, total_rows, first_row);
  }
  return hipGetLastError();
}

}  // namespace commvq
