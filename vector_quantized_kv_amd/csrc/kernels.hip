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

#include <utility>

#include "device_common.h"

namespace commvq {

typedef _Float16 f16;

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return static_cast<float>(*p);
}

// ------------------------------------------------------------------------------------ RoPE table
// One thread per entry, over three sections, each (cos, sin) computed in fp64 and rounded once to fp32: fine
// pair-major (entry j * 64 + f = e^{i f theta_j}), fine group-major (entry ((g * 2 + h) * 64 + f) * 2 + p for
// pair j = 4g + 2h + p: a lane's phases of two pairs in one 16-byte read), coarse position-major (entry
// c * 64 + j = e^{i 64 c theta_j}).
__global__ void __launch_bounds__(256) rope_table_kernel(double base, int64_t n_coarse, float2* out) {
  // theta_j = base^(-2j / head_dim) once per pair and workgroup (64 fp64 pows, not one per entry)
  __shared__ double theta[kPairs];
  if (threadIdx.x < kPairs)
    theta[threadIdx.x] = pow(base, -2.0 * static_cast<int>(threadIdx.x) / static_cast<double>(kHeadDim));
  __syncthreads();
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
    j = 4 * (k >> 8) + 2 * ((k >> 7) & 1) + (k & 1);
    pos = static_cast<double>((k >> 1) & 63);
  } else {
    j = static_cast<int>((idx - 2 * kFine) % kPairs);
    pos = 64.0 * static_cast<double>((idx - 2 * kFine) / kPairs);
  }
  double s, c;
  sincos(pos * theta[j], &s, &c);
  // the sections are contiguous: fine at 0, fine group-major at kRopeFine32gOffset = kFine, coarse after it
  out[idx] = make_float2(static_cast<float>(c), static_cast<float>(s));
}

hipError_t launch_rope_table(double base, int32_t n_positions, float2* table, hipStream_t s) {
  const int64_t n_coarse = rope_coarse_rows(n_positions);
  const int64_t n = 2LL * kFineRows * kPairs + n_coarse * kPairs;
  rope_table_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(base, n_coarse, table);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- query x codebook table
// grid (G*R, Hq, B): the workgroup writes the N x W/2 complex entries of one (b, h, g, r). Byte layout G = 16,
// N = 256, W = 8; bit-packed layout G = 2, N = 64, W = 64. Codeword and entries move in 16-byte pieces (a codeword
// row is W * sizeof(T) >= 16 bytes and 16-byte aligned); consecutive threads take consecutive pieces (thread i:
// piece i mod P of row i / P, P pieces per row), so every wave instruction loads and stores whole contiguous rows.
template <typename T, int W>
constexpr int qtable_pieces = W / (16 / static_cast<int>(sizeof(T)));  // 16-byte pieces per codeword row
template <typename T, int G, int N>
constexpr int qtable_threads = N * qtable_pieces<T, kHeadDim / G> < 256 ? N * qtable_pieces<T, kHeadDim / G> : 256;
template <typename T, int G, int N>
__global__ void __launch_bounds__(256) qtable_kernel(const T* q, const T* kcb, T* out, int Hq, int Hkv, int R) {
  constexpr int W = kHeadDim / G;
  constexpr int kPer = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte piece
  constexpr int P = qtable_pieces<T, W>, kThreads = qtable_threads<T, G, N>;
  static_assert(W % kPer == 0 && (N * P) % kThreads == 0, "codeword rows are whole 16-byte pieces");
  const int gr = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = gr / R, r = gr % R, kv = h / (Hq / Hkv);
  const T* qq = q + (static_cast<int64_t>(b) * Hq + h) * kHeadDim + W * g;
  const uint4* c = reinterpret_cast<const uint4*>(kcb + (((static_cast<int64_t>(kv) * G + g) * R + r) * N) * W);
  uint4* o = reinterpret_cast<uint4*>(out + ((((static_cast<int64_t>(b) * Hq + h) * G + g) * R + r) * N) * W);
#pragma unroll
  for (int it = 0; it < N * P / kThreads; ++it) {
    const int item = static_cast<int>(threadIdx.x) + kThreads * it;  // = row * P + piece
    const int piece = item % P;
    union {
      uint4 v;
      T e[kPer];
    } in, res;
    in.v = c[item];
#pragma unroll
    for (int u = 0; u < kPer / 2; ++u) {
      const int d = piece * kPer + 2 * u;
      const float q0 = ld(qq + d), q1 = ld(qq + d + 1);
      const float a = static_cast<float>(in.e[2 * u]), bb = static_cast<float>(in.e[2 * u + 1]);
      res.e[2 * u] = static_cast<T>(q0 * a + q1 * bb);
      res.e[2 * u + 1] = static_cast<T>(q0 * bb - q1 * a);
    }
    o[item] = res.v;
  }
}

hipError_t launch_qtable(int dtype, bool packed, int R, int B, int Hq, int Hkv, const void* q, const void* kcb,
                         void* out, hipStream_t s) {
  if (packed) {  // fp16 only
    qtable_kernel<f16, kWideGroups, kWideCodes>
        <<<dim3(kWideGroups * R, Hq, B), qtable_threads<f16, kWideGroups, kWideCodes>, 0, s>>>(
            static_cast<const f16*>(q), static_cast<const f16*>(kcb), static_cast<f16*>(out), Hq, Hkv, R);
    return hipGetLastError();
  }
  dim3 grid(kGroups * R, Hq, B);
  if (dtype == COMMVQ_F16)
    qtable_kernel<f16, kGroups, kCodes><<<grid, qtable_threads<f16, kGroups, kCodes>, 0, s>>>(
        static_cast<const f16*>(q), static_cast<const f16*>(kcb), static_cast<f16*>(out), Hq, Hkv, R);
  else
    qtable_kernel<float, kGroups, kCodes><<<grid, qtable_threads<float, kGroups, kCodes>, 0, s>>>(
        static_cast<const float*>(q), static_cast<const float*>(kcb), static_cast<float*>(out), Hq, Hkv, R);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------- value bins
// Fixed-point bins: LDS float atomics are slow on this chip, integer ones are not. Per (work item, head) the
// weights are scaled by a power of two, fx_scale = 2^(B - e) with max|w| < 2^e, so |rint(w * fx_scale)| <= 2^B,
// and a work item of 2^(30 - B) tokens keeps every bin sum within 2^30 (inside int32): B = 18 for the 4096-token
// items of the byte layout in fp16 storage, B = 19 for the 2048-token items of fp32 storage and of the bit-packed
// layout. Pass 0 bins rint(w * fx_scale); the fp32 path adds pass 1, which bins
// rint((w * fx_scale - rint(w * fx_scale)) * 2^(B + 1)), the rounding residual of pass 0 at 2^(B + 1) times the
// resolution (at most 2^B in magnitude; every step exact, as the scales are powers of two). A weight is thus
// represented to 2^-(B + 1) of the item's max|w| (fp16 storage) or 2^-(2B + 2) (fp32). bins layout
// [kGqa][kGroups][R][kCodes].
// Tokens per (sequence, KV head) work item and the fixed-point bits B, by storage type of the byte layout (the
// fp32 kernel keeps 2048-token items: at 4096 its registers spill).
template <typename T>
constexpr int kVrItemTokens = sizeof(T) == 2 ? 2 * kSplitTokens : kSplitTokens;
template <typename T>
constexpr int kVrBits = sizeof(T) == 2 ? 18 : 19;
constexpr int kVrBitsPacked = 19;  // bit-packed layout: 2048-token items
static_assert((static_cast<int64_t>(kVrItemTokens<f16>) << kVrBits<f16>) <= (int64_t{1} << 30) &&
                  (static_cast<int64_t>(kVrItemTokens<float>) << kVrBits<float>) <= (int64_t{1} << 30) &&
                  (static_cast<int64_t>(kSplitTokens) << kVrBitsPacked) <= (int64_t{1} << 30),
              "bin sums stay within 2^30");
template <int kBits>
__device__ __forceinline__ int32_t fixed_point(float w, float fx_scale, int pass) {
  const float x = w * fx_scale;
  const float hi = rintf(x);
  return static_cast<int32_t>(pass == 0 ? hi : rintf((x - hi) * static_cast<float>(1 << (kBits + 1))));
}

template <int kBits>
__device__ __forceinline__ float fixed_point_scale(float max_abs) {
  if (!(max_abs > 0.f)) return 1.f;
  int e;
  frexpf(max_abs, &e);  // max_abs = m 2^e, m in [0.5, 1)
  return ldexpf(1.f, kBits - e);
}

template <int R, int TPT, int kBits>
__device__ __forceinline__ void bin_weights(int32_t* bins, const uint4 (&vc)[TPT][R], const float (&w)[TPT][kGqa],
                                            const bool (&valid)[TPT], const float (&fx_scale)[kGqa], int pass) {
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    if (!valid[k]) continue;
    int32_t fx[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) fx[h] = fixed_point<kBits>(w[k][h], fx_scale[h], pass);
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

// Non-negative weights (a softmax's, the usual case): two heads share a 64-bit bin, layout [2 head pairs][kGroups]
// [R][kCodes] (the same bytes as the int32 bins). A bin's sums stay within 2^30 (see fixed_point_scale), so the
// low head never carries into the high one and one ds_add_u64 does the work of two ds_add_u32.
template <int R, int TPT, int kBits>
__device__ __forceinline__ void bin_weights_pairs(unsigned long long* bins, const uint4 (&vc)[TPT][R],
                                                  const float (&w)[TPT][kGqa], const bool (&valid)[TPT],
                                                  const float (&fx_scale)[kGqa]) {
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    if (!valid[k]) continue;
    uint32_t fx[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) fx[h] = static_cast<uint32_t>(fixed_point<kBits>(w[k][h], fx_scale[h], 0));
    const unsigned long long p01 = fx[0] | (static_cast<unsigned long long>(fx[1]) << 32);
    const unsigned long long p23 = fx[2] | (static_cast<unsigned long long>(fx[3]) << 32);
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t l = code_index(vc[k][r], g);
        __hip_atomic_fetch_add(bins + (g * R + r) * kCodes + l, p01, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(bins + ((kGroups + g) * R + r) * kCodes + l, p23, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
      }
  }
}

// acc[i] += weight * sum_r sum_l bins[h][g][r][l] * CV[g][r][l][w] for output d = (tid + NT i) & 127 of head
// h = (tid + NT i) >> 7 (o = 8 g + w); each of the NT threads handles kGqa * kHeadDim / NT outputs.
template <typename T, int R, int NT>
__device__ __forceinline__ void contract_bins(const int32_t* bins, const T* vcb, float weight,
                                              float (&acc)[kGqa * kHeadDim / NT]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kGqa * kHeadDim / NT; ++i) {
    const int idx = tid + NT * i, h = idx >> 7, d = idx & 127, g = d >> 3, w = d & 7;
    float sum = 0.f;
    for (int r = 0; r < R; ++r) {
      const int32_t* bb = bins + ((h * kGroups + g) * R + r) * kCodes;
      const T* cv = vcb + ((static_cast<int64_t>(g) * R + r) * kCodes) * kGroupDim + w;
      for (int l = 0; l < kCodes; ++l) sum = fmaf(static_cast<float>(bb[l]), ld(cv + l * kGroupDim), sum);
    }
    acc[i] = fmaf(sum, weight, acc[i]);
  }
}

// fp16 storage: the same product on the matrix core (v_mfma_f32_4x4x4_16b_f16). Wave w of the kVrWaves takes
// groups kVrGpw w .. kVrGpw w + kVrGpw - 1 (every residual and codeword), so each output belongs to one wave. Per (group, residual,
// 64-codeword chunk c): a coalesced 16-byte load hands lane l the row of codeword 64 c + l (a byte-layout row is
// 16 bytes), an MFMA against the identity turns each 4x4 (codeword x dim) quad tile into the B operand (lane
// 4 q + j: dim j of codewords 64 c + 4 q .. + 3, exact in fp32, so exact back in fp16), and the bins of head
// h = lane & 3 and those codewords, scaled by 2^-16 (exact: |bin| < 2^31) and split into fp16 hi + lo (2^-22
// relative), are the A operand. The 16 quads of each output are summed across lanes at the end; lane j < 4 then
// writes dims 8 g + 4 x + j of every head: part[h][8 g + 4 x + j] = sum * 2^16 * scale[h].
constexpr int kVrWaves = 8;                      // waves per value-reduce workgroup (one workgroup per CU: the bins)
constexpr int kVrThreads = 64 * kVrWaves;
constexpr int kVrGpw = kGroups / kVrWaves;         // groups per wave in the contraction
static_assert(kGroups % kVrWaves == 0 && kSplitTokens % kVrThreads == 0, "groups and tokens split evenly");
typedef _Float16 vr_h4 __attribute__((ext_vector_type(4)));
typedef float vr_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ vr_f4 vr_mfma(vr_h4 a, vr_h4 b, vr_f4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ vr_h4 vr_row_half(uint32_t x, uint32_t y) {
  const vr_h4 v = {__builtin_bit_cast(f16, static_cast<uint16_t>(x)), __builtin_bit_cast(f16, static_cast<uint16_t>(x >> 16)),
                   __builtin_bit_cast(f16, static_cast<uint16_t>(y)), __builtin_bit_cast(f16, static_cast<uint16_t>(y >> 16))};
  return v;
}
// The wave's codeword rows, rows[gi][r][c] = codeword 64 c + lane of residual r, group kVrGpw wave + gi (loaded
// before the bins are filled, so that their latency hides behind the binning).
template <int R>
__device__ __forceinline__ void load_value_rows(const f16* vcb, uint4 (&rows)[kVrGpw][R][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int gi = 0; gi < kVrGpw; ++gi)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        rows[gi][r][c] = *reinterpret_cast<const uint4*>(
            vcb + ((static_cast<int64_t>(kVrGpw * wave + gi) * R + r) * kCodes + 64 * c + lane) * kGroupDim);
}
template <int R, bool kPairs>
__device__ __forceinline__ void contract_bins_mfma(const int32_t* bins, const uint4 (&rows)[kVrGpw][R][4],
                                                   const float (&scale)[kGqa], float* part, int64_t row_stride) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane & 3, q4 = (lane >> 2) * 4;
  const vr_h4 ident = {static_cast<f16>(hh == 0), static_cast<f16>(hh == 1), static_cast<f16>(hh == 2),
                       static_cast<f16>(hh == 3)};
  const vr_f4 z = {0.f, 0.f, 0.f, 0.f};
  vr_f4 O[kVrGpw][2];
#pragma unroll
  for (int gi = 0; gi < kVrGpw; ++gi) O[gi][0] = O[gi][1] = z;
#pragma unroll
  for (int gi = 0; gi < kVrGpw; ++gi) {
    const int g = kVrGpw * wave + gi;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4 (&row)[4] = rows[gi][r];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int32_t cnt[4];
        if constexpr (kPairs) {  // 64-bit bins of head pair hh / 2: this head is the low or high half
          const int4* bp = reinterpret_cast<const int4*>(
              bins + 2 * (((hh >> 1) * kGroups + g) * R + r) * kCodes + 2 * (64 * c + q4));
          const int4 b0 = bp[0], b1 = bp[1];
          const bool hi = hh & 1;
          cnt[0] = hi ? b0.y : b0.x;
          cnt[1] = hi ? b0.w : b0.z;
          cnt[2] = hi ? b1.y : b1.x;
          cnt[3] = hi ? b1.w : b1.z;
        } else {
          const int4 bq = *reinterpret_cast<const int4*>(bins + ((hh * kGroups + g) * R + r) * kCodes + 64 * c + q4);
          cnt[0] = bq.x;
          cnt[1] = bq.y;
          cnt[2] = bq.z;
          cnt[3] = bq.w;
        }
        vr_h4 ahi, alo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = static_cast<float>(cnt[k]) * (1.f / 65536.f);
          const f16 hi = static_cast<f16>(x);
          ahi[k] = hi;
          alo[k] = static_cast<f16>(x - static_cast<float>(hi));
        }
        const vr_f4 t0 = vr_mfma(vr_row_half(row[c].x, row[c].y), ident, z);
        const vr_f4 t1 = vr_mfma(vr_row_half(row[c].z, row[c].w), ident, z);
        const vr_h4 v0 = {static_cast<f16>(t0[0]), static_cast<f16>(t0[1]), static_cast<f16>(t0[2]), static_cast<f16>(t0[3])};
        const vr_h4 v1 = {static_cast<f16>(t1[0]), static_cast<f16>(t1[1]), static_cast<f16>(t1[2]), static_cast<f16>(t1[3])};
        O[gi][0] = vr_mfma(ahi, v0, O[gi][0]);
        O[gi][0] = vr_mfma(alo, v0, O[gi][0]);
        O[gi][1] = vr_mfma(ahi, v1, O[gi][1]);
        O[gi][1] = vr_mfma(alo, v1, O[gi][1]);
      }
    }
  }
  // sum the 16 quads (lanes with the same j = lane & 3), then lane j writes dim 4 x + j of its groups
#pragma unroll
  for (int gi = 0; gi < kVrGpw; ++gi)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        float v = O[gi][x][h];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane < 4) part[h * row_stride + 4 + 8 * (kVrGpw * wave + gi) + 4 * x + lane] = v * 65536.f * scale[h];
      }
}

// ----------------------------------------------------------------------------------- value reduce
// The reordered value reduce of the pages: weights are binned by value code (bin_weights), then the
// bins are contracted with the value codebook (contract_bins). One workgroup per (sequence, KV head, work item
// of kVrItemTokens tokens: 4096 for fp16 storage, so a 128K context with 8 KV heads fills the 256 CUs in one
// round, the bins taking a CU's LDS); partial outputs, one per item in the first slots of the 2048-token split
// partials, are summed by combine_sum_kernel. Any finite weights bin exactly up to the fixed-point resolution
// above (one pass for fp16 storage, two for fp32).
template <typename T, int R>
__global__ void __launch_bounds__(kVrThreads) value_reduce_kernel(const ValueReduceArgs a) {
  constexpr int kItem = kVrItemTokens<T>, kBits = kVrBits<T>;
  constexpr int TPT = kItem / kVrThreads;
  constexpr int kPasses = sizeof(T) == 4 ? 2 : 1;
  __shared__ float red[kVrWaves][kGqa];
  __shared__ __attribute__((aligned(16))) int32_t work[kGqa * kGroups * R * kCodes];
  const int item = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.p_stride, a.total_tokens);
  const int L = sb.len;
  const int t0 = item * kItem;
  if (t0 >= L) return;
  const int64_t row0 = sb.start + t0;
  const int h0 = kv * kGqa;
  const int wave = tid >> 6, lane = tid & 63;
  bool valid[TPT];
  float w[TPT][kGqa];
  uint4 vc[TPT][R];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = t0 + tid + kVrThreads * k;
    valid[k] = t < L;
#pragma unroll
    for (int h = 0; h < kGqa; ++h)
      w[k][h] = valid[k] ? a.p[(static_cast<int64_t>(b) * a.n_q_heads + h0 + h) * a.p_stride + t] : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
      vc[k][r] = valid[k] ? load_code_record(a.v_codes, a.total_tokens, kv, row0 + tid + kVrThreads * k, R, r)
                          : make_uint4(0, 0, 0, 0);
  }
  __shared__ int neg_w[kVrWaves];
  bool neg = false;
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      mx = fmaxf(mx, fabsf(w[k][h]));
      neg |= w[k][h] < 0.f;
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave][h] = mx;
  }
  const bool wave_neg = __ballot(neg) != 0;
  if (lane == 0) neg_w[wave] = wave_neg;
  __syncthreads();
  bool any_neg = false;
#pragma unroll
  for (int v = 0; v < kVrWaves; ++v) any_neg |= neg_w[v] != 0;
  float fx_scale[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = red[0][h];
#pragma unroll
    for (int v = 1; v < kVrWaves; ++v) mx = fmaxf(mx, red[v][h]);
    fx_scale[h] = fixed_point_scale<kBits>(mx);
  }
  const T* vcb = static_cast<const T*>(a.v_cb) + static_cast<int64_t>(kv) * kGroups * R * kCodes * kGroupDim;
  float* part = a.part + ((static_cast<int64_t>(b) * a.n_q_heads + h0) * a.n_splits + item) * kPartFloats;
  const int64_t row_stride = static_cast<int64_t>(a.n_splits) * kPartFloats;
  if constexpr (sizeof(T) == 2) {
    uint4 rows[kVrGpw][R][4];
    load_value_rows<R>(reinterpret_cast<const f16*>(vcb), rows);
    for (int i = tid; i < kGqa * kGroups * R * kCodes / 4; i += kVrThreads)
      reinterpret_cast<int4*>(work)[i] = make_int4(0, 0, 0, 0);
    __syncthreads();
    float inv[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) inv[h] = 1.f / fx_scale[h];  // a power of two: exact
    if (!any_neg) {
      bin_weights_pairs<R, TPT, kBits>(reinterpret_cast<unsigned long long*>(work), vc, w, valid, fx_scale);
      __syncthreads();
      contract_bins_mfma<R, true>(work, rows, inv, part, row_stride);
    } else {
      bin_weights<R, TPT, kBits>(work, vc, w, valid, fx_scale, 0);
      __syncthreads();
      contract_bins_mfma<R, false>(work, rows, inv, part, row_stride);
    }
  } else {
    constexpr int kOut = kGqa * kHeadDim / kVrThreads;
    float acc[kOut] = {};
    for (int pass = 0; pass < kPasses; ++pass) {
      if (pass > 0) __syncthreads();  // every thread has finished reading the previous pass's bins
      for (int i = tid; i < kGqa * kGroups * R * kCodes / 4; i += kVrThreads)
      reinterpret_cast<int4*>(work)[i] = make_int4(0, 0, 0, 0);
      __syncthreads();
      bin_weights<R, TPT, kBits>(work, vc, w, valid, fx_scale, pass);
      __syncthreads();
      contract_bins<T, R, kVrThreads>(work, vcb, pass == 0 ? 1.f : 1.f / static_cast<float>(1 << (kBits + 1)), acc);
    }
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int idx = tid + kVrThreads * i, h = idx >> 7, d = idx & 127;
      part[h * row_stride + 4 + d] = acc[i] / fx_scale[h];
    }
  }
}

// One workgroup per (b, q head): thread (d, k) sums the work items k, k + 8, ... of output d (four loads in
// flight), and the 8 partial sums are added in a fixed order. A work item covers item_tokens tokens and its partial
// sits in slot item of the partials.
constexpr int kCombineParts = 8;
__global__ void __launch_bounds__(kCombineParts * kHeadDim) combine_sum_kernel(const float* part, const ValueReduceArgs a,
                                                                             int item_tokens, float* out) {
  __shared__ float red[kCombineParts][kHeadDim];
  const int bh = blockIdx.x, b = bh / a.n_q_heads, d = threadIdx.x & (kHeadDim - 1), k = threadIdx.x / kHeadDim;
  const int L = seq_bounds(a.seq_start, a.seq_len, b, a.p_stride, a.total_tokens).len;  // as value_reduce_kernel
  const int n_splits = a.n_splits;
  const int ns = (L + item_tokens - 1) / item_tokens;
  const float* p = part + static_cast<int64_t>(bh) * n_splits * kPartFloats + 4 + d;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int s = k;
  for (; s + 3 * kCombineParts < ns; s += 4 * kCombineParts) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += p[static_cast<int64_t>(s + u * kCombineParts) * kPartFloats];
  }
  for (; s < ns; s += kCombineParts) acc[0] += p[static_cast<int64_t>(s) * kPartFloats];
  red[k][d] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (k == 0) {
    float t = red[0][d];
#pragma unroll
    for (int j = 1; j < kCombineParts; ++j) t += red[j][d];
    out[static_cast<int64_t>(bh) * kHeadDim + d] = t;
  }
}

// Bit-packed records (2 groups of 64 dims, 64 codewords, R <= 32): the same split, fixed point, sign test and
// partials as value_reduce_kernel. A token's indices are read in windows of 8 residuals (3 words, 16 indices).
// Bins [4 heads][2][R][64] int32, or for non-negative splits [2 head pairs][2][R][64] uint64 in the same bytes
// (64 KiB at R = 32: two workgroups share a CU). The contraction runs on the VALU: the R x 64 (residual,
// codeword) rows are dealt evenly to the waves, lane (g, w) accumulates dims 2w, 2w + 1 of group g for the 4
// heads, and the waves' sums meet in LDS (over the bins, once every wave has read them).
template <int F, bool kPairs>
__device__ __forceinline__ void bin_packed_field(int32_t* bins, int R, int c, uint32_t x0, uint32_t x1, uint32_t x2,
                                                 const uint32_t (&fx)[kGqa]) {
  constexpr int G = kWideGroups, N = kWideCodes, g = F & 1;
  const int r = kWideResPerPass * c + (F >> 1);
  if (r >= R) return;  // fields of the last window past the record
  const uint32_t l = packed_index<F>(x0, x1, x2);
  if constexpr (kPairs) {
    unsigned long long* b64 = reinterpret_cast<unsigned long long*>(bins);
    const unsigned long long p01 = fx[0] | (static_cast<unsigned long long>(fx[1]) << 32);
    const unsigned long long p23 = fx[2] | (static_cast<unsigned long long>(fx[3]) << 32);
    __hip_atomic_fetch_add(b64 + (g * R + r) * N + l, p01, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add(b64 + ((G + g) * R + r) * N + l, p23, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
#pragma unroll
    for (int h = 0; h < kGqa; ++h) atomicAdd(&bins[((h * G + g) * R + r) * N + l], static_cast<int32_t>(fx[h]));
  }
}

template <bool kPairs, int... F>
__device__ __forceinline__ void bin_packed_window(int32_t* bins, int R, int c, uint32_t x0, uint32_t x1, uint32_t x2,
                                                  const uint32_t (&fx)[kGqa], std::integer_sequence<int, F...>) {
  (bin_packed_field<F, kPairs>(bins, R, c, x0, x1, x2, fx), ...);
}

// Every record word a thread needs (TPT tokens x NWIN windows x 3 words) is requested before the first add, so
// the HBM latency is paid once per thread.
template <bool kPairs, int TPT, int NWIN>
__device__ __forceinline__ void bin_packed_tokens(int32_t* bins, int R, const uint32_t* rec, int64_t plane,
                                                  const float (&w)[TPT][kGqa], const bool (&valid)[TPT],
                                                  const float (&fx_scale)[kGqa]) {
  const int Wd = wide_record_words(R);
  uint32_t x[TPT][NWIN][3];
#pragma unroll
  for (int k = 0; k < TPT; ++k)
#pragma unroll
    for (int c = 0; c < NWIN; ++c)
#pragma unroll
      for (int i = 0; i < 3; ++i)
        x[k][c][i] = valid[k] ? rec[kVrThreads * k + min(packed_window_word(c) + i, Wd - 1) * plane] : 0u;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    if (!valid[k]) continue;
    uint32_t fx[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) fx[h] = static_cast<uint32_t>(fixed_point<kVrBitsPacked>(w[k][h], fx_scale[h], 0));
#pragma unroll
    for (int c = 0; c < NWIN; ++c)
      bin_packed_window<kPairs>(bins, R, c, x[k][c][0], x[k][c][1], x[k][c][2], fx,
                                std::make_integer_sequence<int, kWideGroups * kWideResPerPass>{});
  }
}

template <bool kPairs, int TPT>
__device__ __forceinline__ void bin_packed_split(int32_t* bins, int R, const uint32_t* rec, int64_t plane,
                                                 const float (&w)[TPT][kGqa], const bool (&valid)[TPT],
                                                 const float (&fx_scale)[kGqa]) {
  static_assert(kWideMaxResiduals == 4 * kWideResPerPass, "at most 4 windows");
  switch ((R + kWideResPerPass - 1) / kWideResPerPass) {
    case 1: bin_packed_tokens<kPairs, TPT, 1>(bins, R, rec, plane, w, valid, fx_scale); break;
    case 2: bin_packed_tokens<kPairs, TPT, 2>(bins, R, rec, plane, w, valid, fx_scale); break;
    case 3: bin_packed_tokens<kPairs, TPT, 3>(bins, R, rec, plane, w, valid, fx_scale); break;
    default: bin_packed_tokens<kPairs, TPT, 4>(bins, R, rec, plane, w, valid, fx_scale); break;
  }
}

// Lane (g, w)'s sums over 8 consecutive (residual, codeword) rows kk .. kk + 7 of the 4 heads.
template <bool kPairs>
__device__ __forceinline__ void contract_packed_rows(const int32_t* bins, int K, int g, int kk,
                                                     const uint32_t (&cv)[8], float (&acc)[kGqa][2]) {
  const unsigned long long* b64 = reinterpret_cast<const unsigned long long*>(bins);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float cnt[kGqa];
    if constexpr (kPairs) {
      const unsigned long long lo = b64[g * K + kk + j], hi = b64[(kWideGroups + g) * K + kk + j];
      cnt[0] = static_cast<float>(static_cast<uint32_t>(lo));
      cnt[1] = static_cast<float>(static_cast<uint32_t>(lo >> 32));
      cnt[2] = static_cast<float>(static_cast<uint32_t>(hi));
      cnt[3] = static_cast<float>(static_cast<uint32_t>(hi >> 32));
    } else {
#pragma unroll
      for (int h = 0; h < kGqa; ++h) cnt[h] = static_cast<float>(bins[(h * kWideGroups + g) * K + kk + j]);
    }
    union {
      uint32_t u;
      f16 e[2];
    } c;
    c.u = cv[j];
    const float c0 = static_cast<float>(c.e[0]), c1 = static_cast<float>(c.e[1]);
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      acc[h][0] = fmaf(cnt[h], c0, acc[h][0]);
      acc[h][1] = fmaf(cnt[h], c1, acc[h][1]);
    }
  }
}

// Rows [k0, k1) (multiples of 8) of the contraction; the codebook words of the next 8 rows are in flight while
// the current 8 are summed.
template <bool kPairs>
__device__ __forceinline__ void contract_packed(const int32_t* bins, int K, int g, int k0, int k1, const f16* vcb,
                                                float (&acc)[kGqa][2]) {
  constexpr int W = kHeadDim / kWideGroups;
  uint32_t cur[8], nxt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cur[j] = *reinterpret_cast<const uint32_t*>(vcb + static_cast<int64_t>(k0 + j) * W);
  for (int kk = k0; kk < k1; kk += 8) {
    const int kn = kk + 8 < k1 ? kk + 8 : kk;  // the last step reloads its own rows (in bounds, unused)
#pragma unroll
    for (int j = 0; j < 8; ++j) nxt[j] = *reinterpret_cast<const uint32_t*>(vcb + static_cast<int64_t>(kn + j) * W);
    contract_packed_rows<kPairs>(bins, K, g, kk, cur, acc);
#pragma unroll
    for (int j = 0; j < 8; ++j) cur[j] = nxt[j];
  }
}

__global__ void __launch_bounds__(kVrThreads) value_reduce_bits_kernel(const ValueReduceArgs a, int R) {
  constexpr int TPT = kSplitTokens / kVrThreads;
  constexpr int G = kWideGroups, N = kWideCodes, W = kHeadDim / G;
  static_assert(G * W / 2 == 64 && kGqa * kHeadDim == kVrThreads, "lane (g, w) pairs and one output per thread");
  __shared__ float red[kVrWaves][kGqa];
  __shared__ int neg_w[kVrWaves];
  __shared__ __attribute__((aligned(16))) int32_t bins[kGqa * G * kWideMaxResiduals * N];
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.p_stride, a.total_tokens);
  const int L = sb.len;
  const int t0 = split * kSplitTokens;
  if (t0 >= L) return;
  const int64_t row0 = sb.start + t0;
  const int h0 = kv * kGqa;
  const int wave = tid >> 6, lane = tid & 63;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(a.v_codes);
  bool valid[TPT];
  float w[TPT][kGqa];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = t0 + tid + kVrThreads * k;
    valid[k] = t < L;
#pragma unroll
    for (int h = 0; h < kGqa; ++h)
      w[k][h] = valid[k] ? a.p[(static_cast<int64_t>(b) * a.n_q_heads + h0 + h) * a.p_stride + t] : 0.f;
  }
  const int n_bins = kGqa * G * R * N;  // a multiple of 4 int32
  for (int i = tid; i < n_bins / 4; i += kVrThreads) reinterpret_cast<int4*>(bins)[i] = make_int4(0, 0, 0, 0);
  bool neg = false;
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      mx = fmaxf(mx, fabsf(w[k][h]));
      neg |= w[k][h] < 0.f;
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave][h] = mx;
  }
  const bool wave_neg = __ballot(neg) != 0;
  if (lane == 0) neg_w[wave] = wave_neg;
  __syncthreads();
  bool any_neg = false;
#pragma unroll
  for (int v = 0; v < kVrWaves; ++v) any_neg |= neg_w[v] != 0;
  float fx_scale[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = 0.f;
#pragma unroll
    for (int v = 0; v < kVrWaves; ++v) mx = fmaxf(mx, red[v][h]);
    fx_scale[h] = fixed_point_scale<kVrBitsPacked>(mx);
  }
  const uint32_t* rec = words + static_cast<int64_t>(kv) * wide_record_words(R) * a.total_tokens + row0 + tid;
  if (!any_neg)
    bin_packed_split<true, TPT>(bins, R, rec, a.total_tokens, w, valid, fx_scale);
  else
    bin_packed_split<false, TPT>(bins, R, rec, a.total_tokens, w, valid, fx_scale);
  __syncthreads();
  // contraction: wave v takes rows [v K / 8, (v + 1) K / 8) of the K = R x 64 (residual, codeword) rows
  const int g = lane >> 5, wp = lane & 31;
  const f16* vcb = static_cast<const f16*>(a.v_cb) + static_cast<int64_t>(kv) * G * R * N * W + g * R * N * W + 2 * wp;
  const int K = R * N, k0 = wave * K / kVrWaves, k1 = (wave + 1) * K / kVrWaves;
  float acc[kGqa][2] = {};
  static_assert(kWideCodes % (8 * kVrWaves) == 0, "each wave's rows are whole steps of 8");
  if (!any_neg)
    contract_packed<true>(bins, K, g, k0, k1, vcb, acc);
  else
    contract_packed<false>(bins, K, g, k0, k1, vcb, acc);
  __syncthreads();  // every wave has read the bins: their LDS takes the waves' sums
  float* sums = reinterpret_cast<float*>(bins);  // [kVrWaves][kGqa][kHeadDim], 16 KiB
#pragma unroll
  for (int h = 0; h < kGqa; ++h)
    *reinterpret_cast<float2*>(sums + (wave * kGqa + h) * kHeadDim + W * g + 2 * wp) = make_float2(acc[h][0], acc[h][1]);
  __syncthreads();
  const int h = tid >> 7, d = tid & (kHeadDim - 1);
  float o = 0.f;
#pragma unroll
  for (int v = 0; v < kVrWaves; ++v) o += sums[(v * kGqa + h) * kHeadDim + d];
  float* part = a.part + ((static_cast<int64_t>(b) * a.n_q_heads + h0) * a.n_splits + split) * kPartFloats;
  const int64_t row_stride = static_cast<int64_t>(a.n_splits) * kPartFloats;
  part[h * row_stride + 4 + d] = o / fx_scale[h];
}

hipError_t launch_value_reduce(int dtype, bool packed, int R, int B, const ValueReduceArgs& a, float* out,
                               hipStream_t s) {
  // work items: 2048-token splits (bit-packed, byte layout in fp32), pairs of them (byte layout in fp16)
  const int item_tokens = packed ? kSplitTokens : (dtype == COMMVQ_F16 ? kVrItemTokens<f16> : kVrItemTokens<float>);
  dim3 grid((a.n_splits * kSplitTokens + item_tokens - 1) / item_tokens, a.n_kv_heads, B);
  if (packed) {  // fp16 only
    value_reduce_bits_kernel<<<grid, kVrThreads, 0, s>>>(a, R);
  } else if (dtype == COMMVQ_F16) {
    if (R == 1) value_reduce_kernel<f16, 1><<<grid, kVrThreads, 0, s>>>(a);
    else value_reduce_kernel<f16, 2><<<grid, kVrThreads, 0, s>>>(a);
  } else {
    if (R == 1) value_reduce_kernel<float, 1><<<grid, kVrThreads, 0, s>>>(a);
    else value_reduce_kernel<float, 2><<<grid, kVrThreads, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_sum_kernel<<<dim3(B * a.n_q_heads), dim3(kCombineParts * kHeadDim), 0, s>>>(a.part, a, item_tokens, out);
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

// Bit-packed records: one thread per (kv, token, window c); it reads the window's three words and unpacks
// them with the same window functions the attention kernel uses. out is [Hkv][R][T][2] int32.
__global__ void debug_unpack_bits_kernel(const uint32_t* words, int64_t total_tokens, int R, int Wd, int n_windows,
                                         int64_t n_items, int32_t* out) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= n_items) return;
  const int c = static_cast<int>(item % n_windows);
  const int64_t kt = item / n_windows;  // kv * T + t
  const int64_t kv = kt / total_tokens, t = kt % total_tokens;
  const uint32_t* rec = words + kv * Wd * total_tokens + t;  // word w at rec[w * total_tokens]
  const int w0 = packed_window_word(c);
  const uint32_t x0 = rec[min(w0, Wd - 1) * total_tokens], x1 = rec[min(w0 + 1, Wd - 1) * total_tokens];
  const uint32_t x2 = rec[min(w0 + 2, Wd - 1) * total_tokens];
  static_assert(kWideResPerPass == 8 && kWideGroups == 2, "sixteen indices per window");
  const uint32_t idx[2 * kWideResPerPass] = {
      packed_index<0>(x0, x1, x2),  packed_index<1>(x0, x1, x2),  packed_index<2>(x0, x1, x2),
      packed_index<3>(x0, x1, x2),  packed_index<4>(x0, x1, x2),  packed_index<5>(x0, x1, x2),
      packed_index<6>(x0, x1, x2),  packed_index<7>(x0, x1, x2),  packed_index<8>(x0, x1, x2),
      packed_index<9>(x0, x1, x2),  packed_index<10>(x0, x1, x2), packed_index<11>(x0, x1, x2),
      packed_index<12>(x0, x1, x2), packed_index<13>(x0, x1, x2), packed_index<14>(x0, x1, x2),
      packed_index<15>(x0, x1, x2)};
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
// pass stores every word, group 1's pass ORs its fields into them (ceil(12 R / 32) words per token, one in
// each word plane, so consecutive tokens store consecutive words).
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
  uint32_t* rec = words + static_cast<int64_t>(kv) * Wd * total_rows + first_row + tt;  // word w at rec[w * total_rows]
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
        if (g > 0) v |= rec[word * total_rows];
        rec[word * total_rows] = v;
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
    const uint32_t* rec = words + static_cast<int64_t>(kv) * Wd * n + t;
    const f16* xv = x + (static_cast<int64_t>(kv) * n + t) * kHeadDim + g * W + s * kUpdSlice;
    double res[kUpdSlice];
#pragma unroll
    for (int w = 0; w < kUpdSlice; ++w) res[w] = static_cast<double>(static_cast<float>(xv[w]));
    for (int r = 0; r < R; ++r) {
      const int l = static_cast<int>(packed_field(rec, n, r, g));
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
