// HIP kernels for CommVQ decode-step attention on gfx950.
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

#include "commvq_internal.h"

namespace commvq {

typedef _Float16 f16;

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return static_cast<float>(*p);
}

// Unpack: byte g of a 16-byte code record is the index of group g (N = 256, one byte per index).
// Every kernel that reads codes goes through this function.
__device__ __forceinline__ uint32_t code_index(const uint4& w, int g) {
  const uint32_t word = (g < 4) ? w.x : (g < 8) ? w.y : (g < 12) ? w.z : w.w;
  return (word >> ((g & 3) * 8)) & 0xffu;
}

__device__ __forceinline__ uint4 load_code_record(const uint8_t* codes, int64_t total_tokens, int kv, int64_t row,
                                                  int R, int r) {
  return *reinterpret_cast<const uint4*>(codes + ((static_cast<int64_t>(kv) * total_tokens + row) * R + r) * 16);
}

// e^{i t theta_j} from the two-level table: coarse[t >> 6][j] * fine[t & 63][j].
__device__ __forceinline__ float2 rope_phase(const float2* rope, int t, int j) {
  const float2 f = rope[(t & 63) * kPairs + j];
  const float2 c = rope[kFineRows * kPairs + (t >> 6) * kPairs + j];
  return make_float2(c.x * f.x - c.y * f.y, c.x * f.y + c.y * f.x);
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

// ------------------------------------------------------------------------------------ RoPE table
__global__ void rope_table_kernel(double base, int64_t n_rows, float2* out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n_rows * kPairs) return;
  const int64_t row = idx / kPairs;
  const int j = static_cast<int>(idx % kPairs);
  const double pos = row < kFineRows ? static_cast<double>(row) : 64.0 * static_cast<double>(row - kFineRows);
  const double theta = pow(base, -2.0 * j / static_cast<double>(kHeadDim));
  double s, c;
  sincos(pos * theta, &s, &c);
  out[idx] = make_float2(static_cast<float>(c), static_cast<float>(s));
}

hipError_t launch_rope_table(double base, int32_t n_positions, float2* table, hipStream_t s) {
  const int64_t rows = kFineRows + rope_coarse_rows(n_positions);
  const int64_t n = rows * kPairs;
  rope_table_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(base, rows, table);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- query x codebook table
// grid (G*R, Hq, B), block 256: thread l writes the 4 complex entries of code l.
template <typename T>
__global__ void __launch_bounds__(256) qtable_kernel(const T* q, const T* kcb, T* out, int Hq, int Hkv, int R) {
  const int gr = blockIdx.x, h = blockIdx.y, b = blockIdx.z, l = threadIdx.x;
  const int g = gr / R, r = gr % R, kv = h / (Hq / Hkv);
  const T* qq = q + (static_cast<int64_t>(b) * Hq + h) * kHeadDim + kGroupDim * g;
  const T* c = kcb + (((static_cast<int64_t>(kv) * kGroups + g) * R + r) * kCodes + l) * kGroupDim;
  T* o = out + ((((static_cast<int64_t>(b) * Hq + h) * kGroups + g) * R + r) * kCodes + l) * kGroupDim;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float q0 = ld(qq + 2 * u), q1 = ld(qq + 2 * u + 1), a = ld(c + 2 * u), bb = ld(c + 2 * u + 1);
    o[2 * u] = static_cast<T>(q0 * a + q1 * bb);
    o[2 * u + 1] = static_cast<T>(q0 * bb - q1 * a);
  }
}

hipError_t launch_qtable(int dtype, int R, int B, int Hq, int Hkv, const void* q, const void* kcb, void* out,
                         hipStream_t s) {
  dim3 grid(kGroups * R, Hq, B);
  if (dtype == COMMVQ_F16)
    qtable_kernel<f16><<<grid, 256, 0, s>>>(static_cast<const f16*>(q), static_cast<const f16*>(kcb),
                                            static_cast<f16*>(out), Hq, Hkv, R);
  else
    qtable_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(q), static_cast<const float*>(kcb),
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

// ------------------------------------------------------------------------------ attention split
// One workgroup per (split of kSplitTokens tokens, KV head, sequence); 256 threads, thread owns tokens
// t0 + tid + 256k. Keys: table-gather scores, group by group: the query x codebook table of the 4 q
// heads for one group is built in LDS, then each token gathers its R entries per pair, rotates by its
// RoPE phase and accumulates Re(.). Split-local softmax. Values: weights binned by code index
// (fixed-point LDS atomics), then bins x value codebook. Writes the partial (m, l, o[128]).
template <typename T, int R>
__global__ void __launch_bounds__(256) attn_split_kernel(const AttnArgs a) {
  constexpr int TPT = kSplitTokens / 256;
  __shared__ float qs[kGqa][kHeadDim];
  __shared__ float red[4][kGqa];
  __shared__ __attribute__((aligned(16))) int32_t work[kGqa * kGroups * R * kCodes];

  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int L = a.seq_len[b];
  const int t0 = split * kSplitTokens;
  if (t0 >= L) return;
  const int64_t row0 = a.seq_start[b] + t0;
  const int h0 = kv * kGqa;
  const int wave = tid >> 6, lane = tid & 63;

  const T* q = static_cast<const T*>(a.q) + (static_cast<int64_t>(b) * a.n_q_heads + h0) * kHeadDim;
  for (int i = tid; i < kGqa * kHeadDim; i += 256) qs[i / kHeadDim][i % kHeadDim] = ld(q + i);

  bool valid[TPT];
  uint4 kc[TPT][R];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    valid[k] = t0 + tid + 256 * k < L;
#pragma unroll
    for (int r = 0; r < R; ++r)
      kc[k][r] = valid[k] ? load_code_record(a.k_codes, a.total_tokens, kv, row0 + tid + 256 * k, R, r)
                          : make_uint4(0, 0, 0, 0);
  }
  float s[TPT][kGqa];
#pragma unroll
  for (int k = 0; k < TPT; ++k)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) s[k][h] = 0.f;

  float2* tile = reinterpret_cast<float2*>(work);  // [kGqa][R][kCodes][4 pairs]
  const T* kcb = static_cast<const T*>(a.k_cb) + static_cast<int64_t>(kv) * kGroups * R * kCodes * kGroupDim;
  __syncthreads();

  for (int g = 0; g < kGroups; ++g) {
    for (int e = tid; e < kGqa * R * kCodes * 4; e += 256) {
      const int u = e & 3, l = (e >> 2) & (kCodes - 1), hr = e >> 10, r = hr % R, h = hr / R;
      const T* c = kcb + ((static_cast<int64_t>(g) * R + r) * kCodes + l) * kGroupDim + 2 * u;
      const float ca = ld(c), cb = ld(c + 1);
      const int j = 4 * g + u;
      const float q0 = qs[h][2 * j], q1 = qs[h][2 * j + 1];
      tile[((h * R + r) * kCodes + l) * 4 + u] = make_float2(q0 * ca + q1 * cb, q0 * cb - q1 * ca);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      if (!valid[k]) continue;
      const int t = t0 + tid + 256 * k;
      uint32_t li[R];
#pragma unroll
      for (int r = 0; r < R; ++r) li[r] = code_index(kc[k][r], g);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float2 ph = rope_phase(a.rope, t, 4 * g + u);
#pragma unroll
        for (int h = 0; h < kGqa; ++h) {
          float xr = 0.f, xi = 0.f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float2 v = tile[((h * R + r) * kCodes + li[r]) * 4 + u];
            xr += v.x;
            xi += v.y;
          }
          s[k][h] += xr * ph.x - xi * ph.y;
        }
      }
    }
    __syncthreads();
  }

  // split-local softmax statistics
  float m[kGqa], lsum[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      s[k][h] *= a.scale;
      if (valid[k]) mx = fmaxf(mx, s[k][h]);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave][h] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kGqa; ++h) m[h] = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      s[k][h] = valid[k] ? expf(s[k][h] - m[h]) : 0.f;
      sum += s[k][h];
    }
    sum = wave_sum(sum);
    if (lane == 0) red[wave][h] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kGqa; ++h) lsum[h] = (red[0][h] + red[1][h]) + (red[2][h] + red[3][h]);

  // value bins
  for (int i = tid; i < kGqa * kGroups * R * kCodes; i += 256) work[i] = 0;
  uint4 vc[TPT][R];
#pragma unroll
  for (int k = 0; k < TPT; ++k)
#pragma unroll
    for (int r = 0; r < R; ++r)
      vc[k][r] = valid[k] ? load_code_record(a.v_codes, a.total_tokens, kv, row0 + tid + 256 * k, R, r)
                          : make_uint4(0, 0, 0, 0);
  float fx_scale[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) fx_scale[h] = 1048576.f;  // weights are in [0, 1]
  __syncthreads();
  bin_weights<R, TPT>(work, vc, s, valid, fx_scale);
  __syncthreads();

  float* part = a.part + ((static_cast<int64_t>(b) * a.n_q_heads + h0) * a.n_splits + split) * kPartFloats;
  const int64_t row_stride = static_cast<int64_t>(a.n_splits) * kPartFloats;
  const T* vcb = static_cast<const T*>(a.v_cb) + static_cast<int64_t>(kv) * kGroups * R * kCodes * kGroupDim;
  contract_bins<T, R>(work, vcb, fx_scale, part, row_stride);
  if (tid < kGqa) {
    part[tid * row_stride + 0] = m[tid];
    part[tid * row_stride + 1] = lsum[tid];
  }
}

// Softmax combine over splits: out = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s.
__global__ void __launch_bounds__(128) combine_softmax_kernel(const float* part, const int32_t* seq_len,
                                                              int32_t n_splits, int32_t Hq, float* out) {
  const int bh = blockIdx.x, b = bh / Hq, d = threadIdx.x;
  const int L = seq_len[b];
  const int ns = (L + kSplitTokens - 1) / kSplitTokens;
  const float* p = part + static_cast<int64_t>(bh) * n_splits * kPartFloats;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, p[s * kPartFloats]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = expf(p[s * kPartFloats] - M);
    den = fmaf(w, p[s * kPartFloats + 1], den);
    num = fmaf(w, p[s * kPartFloats + 4 + d], num);
  }
  out[static_cast<int64_t>(bh) * kHeadDim + d] = ns > 0 ? num / den : 0.f;
}

hipError_t launch_attn(int dtype, int R, int B, const AttnArgs& a, float* out, hipStream_t s) {
  dim3 grid(a.n_splits, a.n_kv_heads, B);
  if (dtype == COMMVQ_F16) {
    if (R == 1) attn_split_kernel<f16, 1><<<grid, 256, 0, s>>>(a);
    else attn_split_kernel<f16, 2><<<grid, 256, 0, s>>>(a);
  } else {
    if (R == 1) attn_split_kernel<float, 1><<<grid, 256, 0, s>>>(a);
    else attn_split_kernel<float, 2><<<grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_softmax_kernel<<<dim3(B * a.n_q_heads), dim3(128), 0, s>>>(a.part, a.seq_len, a.n_splits, a.n_q_heads,
                                                                      out);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------- value reduce
// Same bins + contraction as the attention kernel, with caller weights. Fixed-point scale per head is
// 2^20 / max|p| over the split, so any finite weights bin exactly up to that relative resolution.
template <typename T, int R>
__global__ void __launch_bounds__(256) value_reduce_kernel(const ValueReduceArgs a) {
  constexpr int TPT = kSplitTokens / 256;
  __shared__ float red[4][kGqa];
  __shared__ __attribute__((aligned(16))) int32_t work[kGqa * kGroups * R * kCodes];
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int L = a.seq_len[b];
  const int t0 = split * kSplitTokens;
  if (t0 >= L) return;
  const int64_t row0 = a.seq_start[b] + t0;
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

__global__ void __launch_bounds__(128) combine_sum_kernel(const float* part, const int32_t* seq_len,
                                                          int32_t n_splits, int32_t Hq, float* out) {
  const int bh = blockIdx.x, b = bh / Hq, d = threadIdx.x;
  const int L = seq_len[b];
  const int ns = (L + kSplitTokens - 1) / kSplitTokens;
  const float* p = part + static_cast<int64_t>(bh) * n_splits * kPartFloats;
  float acc = 0.f;
  for (int s = 0; s < ns; ++s) acc += p[s * kPartFloats + 4 + d];
  out[static_cast<int64_t>(bh) * kHeadDim + d] = acc;
}

hipError_t launch_value_reduce(int dtype, int R, int B, const ValueReduceArgs& a, float* out, hipStream_t s) {
  dim3 grid(a.n_splits, a.n_kv_heads, B);
  if (dtype == COMMVQ_F16) {
    if (R == 1) value_reduce_kernel<f16, 1><<<grid, 256, 0, s>>>(a);
    else value_reduce_kernel<f16, 2><<<grid, 256, 0, s>>>(a);
  } else {
    if (R == 1) value_reduce_kernel<float, 1><<<grid, 256, 0, s>>>(a);
    else value_reduce_kernel<float, 2><<<grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_sum_kernel<<<dim3(B * a.n_q_heads), dim3(128), 0, s>>>(a.part, a.seq_len, a.n_splits, a.n_q_heads, out);
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

}  // namespace commvq
