// Decode-step attention over a CommVQ cache on gfx950: one fused kernel per call.
//
// What it computes (sources by page title and section):
//   score_t = scale * sum_j Re( conj(q_j) * khat_{t,j} * e^{i t theta_j} )
//   out     = sum_t softmax(score)_t * vhat_t
// with khat, vhat the additive decodes (sum over R residual codebooks) of the stored code indices
// ("1-bit quantization" tag page, CommVQ abstract; pith.science verdict for arXiv 2506.18879,
// pith_extraction.key_machinery). Because each key codeword block [[a,-b],[b,a]] commutes with the RoPE
// rotation, the rotation by position can be split freely between the query side and the key side; the
// kernel puts the per-64-token part on the query (once per block) and the per-lane part on the keys.
//
// Work item: one workgroup (4 waves) per (sequence b, KV head, split of `split_tokens` tokens). Each wave
// owns 64-token blocks; lane = token within the block, so the fine RoPE phase e^{i (t mod 64) theta_j}
// is a per-lane constant held in registers (64 packed fp16 pairs).
//
// Phases (K residual 0..R-1, then V residual 0..R-1), each over the whole split with the residual's 64 KiB
// codebook in LDS, filled by direct global->LDS loads that overlap the phase's prefetch of code records
// and coarse phases (two workgroups per CU, so one computes while the other waits on its loads):
//   K phase: gather the token's 16 codewords (one ds_read_b128 each), rotate them by the fine phase
//            (2 packed-fp16 ops per pair), and form the 4 GQA head scores with v_mfma_f32_4x4x4_16b_f16:
//            B = the token's rotated key (4 dims per step), A = the query rotated by the conjugate coarse
//            phase of the block, broadcast from one 4-lane block (CBSZ/ABID) so each lane supplies only
//            4 of the 64 query pairs. Scores accumulate across residuals in the MFMA accumulator.
//   softmax: split max / sum over the workgroup; weights p = e^{s - m} in registers.
//   V phase: gather value codewords, transpose each 4x4 (token x dim) tile of a lane quad with an
//            identity-B MFMA, and accumulate p^T x v with the same 4x4x4 MFMA (the reduction over tokens
//            runs inside each quad; the 16 quads are summed once at the end).
// The workgroup writes (m, l, o[128]) per q head; the last workgroup of each (b, kv) (arrival counter in
// the workspace, reset to zero by that workgroup) merges the splits and writes out.
//
// fp32 storage uses the same structure with each fp32 operand split into fp16 hi + lo parts (three MFMA
// products per step), the fine phase read from the table, and a 128 KiB codebook buffer.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>
#include <utility>

#include "device_common.h"

namespace commvq {
namespace {

typedef _Float16 f16;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kAttnThreads / 64;

template <int ABID>
__device__ __forceinline__ f4 mfma_bcast(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}
__device__ __forceinline__ f4 mfma(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0); }

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ h4 cat(h2 a, h2 b) { return (h4){a.x, a.y, b.x, b.y}; }
__device__ __forceinline__ h4 to_h4(f4 x) { return (h4){(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]}; }

// k * e^{i phi} for packed fp16 complex numbers (re in the low half, im in the high half), with
// f = (cos, sin): t = k.im * f = (k.im cos, k.im sin), then w = k.re * f + (-t.im, t.re). Every half
// broadcast, swap and negation applies to k or t (values used once), so they fold into operand
// modifiers of the two packed instructions and f is used as stored.
__device__ __forceinline__ h2 crot(h2 k, h2 f) {
  const h2 t = (h2){k.y, k.y} * f;
  return (h2){k.x, k.x} * f + (h2){-t.y, t.x};
}

struct Split2 {  // fp32 value as fp16 hi + lo
  f16 hi, lo;
};
__device__ __forceinline__ Split2 split2(float x) {
  f16 h = (f16)x;
  return {h, (f16)(x - (float)h)};
}

// Identity B operand: lane 4b+j holds e_j, so D_b = A_b (a quad transpose of A).
__device__ __forceinline__ h4 identity_b(int lane) {
  const int j = lane & 3;
  return (h4){(f16)(j == 0), (f16)(j == 1), (f16)(j == 2), (f16)(j == 3)};
}

// ---------------------------------------------------------------------------------- per-group steps
// Key step for group G of one 64-token block: gather, rotate, two MFMA steps (4 dims each).
template <int G, typename T>
struct KeyGroup;

template <int G>
struct KeyGroup<G, f16> {
  __device__ __forceinline__ static void run(const unsigned char* tab, const uint4& code, const h2 (&F)[kPairs],
                                             const h4& A0, const h4& A1, f4& acc) {
    const uint32_t idx = code_index(code, G);
    const uint4 row = *reinterpret_cast<const uint4*>(tab + G * kCodes * 16 + idx * 16);
    const h2 w0 = crot(as_h2(row.x), F[4 * G + 0]);
    const h2 w1 = crot(as_h2(row.y), F[4 * G + 1]);
    const h2 w2 = crot(as_h2(row.z), F[4 * G + 2]);
    const h2 w3 = crot(as_h2(row.w), F[4 * G + 3]);
    const h4 A = (G < 8) ? A0 : A1;
    acc = mfma_bcast<(2 * G) & 15>(A, cat(w0, w1), acc);
    acc = mfma_bcast<(2 * G + 1) & 15>(A, cat(w2, w3), acc);
  }
};

// fp32: row of 8 floats (32 bytes); rotation in fp32, then hi/lo fp16 parts; three products per step.
template <int G>
struct KeyGroup<G, float> {
  __device__ __forceinline__ static void run(const unsigned char* tab, const uint4& code, const float2* fine,
                                             const h4 (&Ah)[2], const h4 (&Al)[2], f4& acc) {
    const uint32_t idx = code_index(code, G);
    const float4 r0 = *reinterpret_cast<const float4*>(tab + G * kCodes * 32 + idx * 32);
    const float4 r1 = *reinterpret_cast<const float4*>(tab + G * kCodes * 32 + idx * 32 + 16);
    const float kk[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float w[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float2 f = fine[(4 * G + u) * kFineRows];
      w[2 * u] = kk[2 * u] * f.x - kk[2 * u + 1] * f.y;
      w[2 * u + 1] = kk[2 * u] * f.y + kk[2 * u + 1] * f.x;
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      h4 bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const Split2 s = split2(w[4 * st + e]);
        bh[e] = s.hi;
        bl[e] = s.lo;
      }
      const int m = G < 8 ? 0 : 1;
      if (st == 0) {
        acc = mfma_bcast<(2 * G) & 15>(Ah[m], bh, acc);
        acc = mfma_bcast<(2 * G) & 15>(Ah[m], bl, acc);
        acc = mfma_bcast<(2 * G) & 15>(Al[m], bh, acc);
      } else {
        acc = mfma_bcast<(2 * G + 1) & 15>(Ah[m], bh, acc);
        acc = mfma_bcast<(2 * G + 1) & 15>(Ah[m], bl, acc);
        acc = mfma_bcast<(2 * G + 1) & 15>(Al[m], bh, acc);
      }
    }
  }
};

// Value step for group G: gather 8 dims, quad-transpose 2 tiles, accumulate p^T v into O[2G], O[2G+1].
template <int G, typename T>
struct ValueGroup;

template <int G>
struct ValueGroup<G, f16> {
  __device__ __forceinline__ static void run(const unsigned char* tab, const uint4& code, const h4& ident,
                                             const h4& pt, const h4& /*unused*/, f4 (&O)[2 * kGroups]) {
    const uint32_t idx = code_index(code, G);
    const uint4 row = *reinterpret_cast<const uint4*>(tab + G * kCodes * 16 + idx * 16);
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    const f4 x0 = mfma(cat(as_h2(row.x), as_h2(row.y)), ident, z);
    const f4 x1 = mfma(cat(as_h2(row.z), as_h2(row.w)), ident, z);
    O[2 * G] = mfma(pt, to_h4(x0), O[2 * G]);
    O[2 * G + 1] = mfma(pt, to_h4(x1), O[2 * G + 1]);
  }
};

template <int G>
struct ValueGroup<G, float> {
  __device__ __forceinline__ static void run(const unsigned char* tab, const uint4& code, const h4& ident,
                                             const h4& pth, const h4& ptl, f4 (&O)[2 * kGroups]) {
    const uint32_t idx = code_index(code, G);
    const float4 r0 = *reinterpret_cast<const float4*>(tab + G * kCodes * 32 + idx * 32);
    const float4 r1 = *reinterpret_cast<const float4*>(tab + G * kCodes * 32 + idx * 32 + 16);
    const float v[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      h4 vh, vl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const Split2 s = split2(v[4 * c + e]);
        vh[e] = s.hi;
        vl[e] = s.lo;
      }
      const h4 bh = to_h4(mfma(vh, ident, z));  // exact: transposed fp16 values
      const h4 bl = to_h4(mfma(vl, ident, z));
      O[2 * G + c] = mfma(pth, bh, O[2 * G + c]);
      O[2 * G + c] = mfma(pth, bl, O[2 * G + c]);
      O[2 * G + c] = mfma(ptl, bh, O[2 * G + c]);
    }
  }
};

template <typename T, typename... Args, int... Gs>
__device__ __forceinline__ void key_groups(std::integer_sequence<int, Gs...>, Args&&... args) {
  (KeyGroup<Gs, T>::run(args...), ...);
}
template <typename T, typename... Args, int... Gs>
__device__ __forceinline__ void value_groups(std::integer_sequence<int, Gs...>, Args&&... args) {
  (ValueGroup<Gs, T>::run(args...), ...);
}

// Fill one phase's codebook table (16 groups x 256 codes, row = W values of T) in LDS with direct
// global->LDS 16-byte loads; each wave moves its quarter. cb_kv points at codebook [kv][0][0][0][0].
template <typename T, int R>
__device__ __forceinline__ void load_table(const T* cb_kv, int r, unsigned char* dst, int wave, int lane) {
  constexpr int kRowBytes = kGroupDim * sizeof(T);
  constexpr int kChunksPerRow = kRowBytes / 16;
  constexpr int kChunks = kGroups * kCodes * kChunksPerRow;
  constexpr int kPerWave = kChunks / kWaves;
#pragma unroll 4
  for (int i = 0; i < kPerWave / 64; ++i) {
    const int c = wave * kPerWave + i * 64 + lane;
    const int rowi = c / kChunksPerRow, part = c % kChunksPerRow;
    const int g = rowi >> 8, l = rowi & (kCodes - 1);
    const unsigned char* gp =
        reinterpret_cast<const unsigned char*>(cb_kv + ((static_cast<int64_t>(g) * R + r) * kCodes + l) * kGroupDim) +
        part * 16;
    __builtin_amdgcn_global_load_lds(gp, dst + (wave * kPerWave + i * 64) * 16, 16, 0, 0);
  }
}

// row_ror DPP: lane l of each 16-lane row reads lane (l + n) mod 16 of the same row.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf,
                                                               false));
}

constexpr int kMaxBlocks = kAttnMaxBlocksPerWave;

template <typename T, int R>
__global__ void __launch_bounds__(kAttnThreads, (std::is_same<T, float>::value ? 1 : 2))
    attn_kernel(const AttnArgs a) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int kRowBytes = kGroupDim * sizeof(T);
  constexpr int kTableBytes = kGroups * kCodes * kRowBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kTableBytes];
  __shared__ float red[2][kWaves][kGqa];
  __shared__ int is_last;

  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = a.seq_len[b];
  const int S = a.split_tokens;
  const int t0 = split * S;
  const int h0 = kv * kGqa;
  float* out_bh = a.out + (static_cast<int64_t>(b) * a.n_q_heads + h0) * kHeadDim;
  if (t0 >= L) {
    if (split == 0)  // empty sequence: the output is zero
      for (int i = tid; i < kGqa * kHeadDim; i += kAttnThreads) out_bh[i] = 0.f;
    return;
  }
  const int nvalid = min(S, L - t0);
  const int nblocks = (nvalid + 63) >> 6;
  const int my_blocks = (nblocks - wave + kWaves - 1) / kWaves;  // blocks wave, wave+4, ...
  const int64_t row_base = a.seq_start[b] + t0;
  const int64_t cb_stride = static_cast<int64_t>(kGroups) * R * kCodes * kGroupDim;
  const T* cb_k = static_cast<const T*>(a.k_cb) + kv * cb_stride;
  const T* cb_v = static_cast<const T*>(a.v_cb) + kv * cb_stride;

  // token row of block i for this lane, clamped into the split so every prefetch is in bounds
  auto token_row = [&](int i) -> int64_t {
    const int tl = (wave + kWaves * i) * 64 + lane;
    return row_base + min(tl, nvalid - 1);
  };

  // query pairs this lane supplies to the broadcast A operand: head qi, pairs 2*quad + {0,1} (+32)
  const int quad = lane >> 2, qi = lane & 3;
  const T* qp = static_cast<const T*>(a.q) + (static_cast<int64_t>(b) * a.n_q_heads + h0 + qi) * kHeadDim;
  float2 qv[4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 32 * m + 2 * quad + e;
      qv[2 * m + e] = make_float2(static_cast<float>(qp[2 * j]), static_cast<float>(qp[2 * j + 1]));
    }
  const float2* coarse = a.rope + kFineRows * kPairs;
  const float2* fine = a.rope + lane;  // fine[j * 64 + (t mod 64)], t mod 64 = lane: stride kFineRows per pair

  f4 sc[kMaxBlocks];
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) sc[i] = (f4){0.f, 0.f, 0.f, 0.f};

  // Code records of the current phase live in code[]; as soon as a block has consumed its record, the
  // record of the same token for the next phase is requested, so the next phase's codes stream in while
  // this phase computes (phases: K residual 0..R-1, then V residual 0..R-1).
  uint4 code[kMaxBlocks];
  auto request_codes = [&](int ph, int i) {
    const uint8_t* base = ph < R ? a.k_codes : a.v_codes;
    code[i] = load_code_record(base, a.total_tokens, kv, token_row(i), R, ph % R);
  };
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i)
    if (i < my_blocks) request_codes(0, i);

  // ------------------------------------------------------------------------------ key phases
  {
    h2 F[kPairs];
    if constexpr (!kF32) {
#pragma unroll
      for (int j = 0; j < kPairs; ++j) {
        const float2 f = fine[j * kFineRows];
        F[j] = (h2){(f16)f.x, (f16)f.y};
      }
    }
    // A operands: the query rotated by the conjugate coarse phase of each 64-token block,
    // q'' = q * conj(C), in fp16 (fp32 inputs: hi and lo fp16 parts); the same for every key phase.
    h4 Ah[kMaxBlocks][2], Al[kMaxBlocks][2];
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      if (i < my_blocks) {
        const float2* cr = coarse + static_cast<int64_t>((t0 + (wave + kWaves * i) * 64) >> 6) * kPairs;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float4 c = *reinterpret_cast<const float4*>(cr + 32 * m + 2 * quad);
          const float2 q0 = qv[2 * m], q1 = qv[2 * m + 1];
          const float qq[4] = {q0.x * c.x + q0.y * c.y, q0.y * c.x - q0.x * c.y, q1.x * c.z + q1.y * c.w,
                               q1.y * c.z - q1.x * c.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const Split2 sp = split2(qq[e]);
            Ah[i][m][e] = sp.hi;
            Al[i][m][e] = sp.lo;
          }
        }
      }
    }
    for (int r = 0; r < R; ++r) {
      if (r > 0) __syncthreads();  // every wave is done with the previous table
      load_table<T, R>(cb_k, r, lds, wave, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kMaxBlocks; ++i) {
        if (i < my_blocks) {
          if constexpr (!kF32) {
            key_groups<f16>(std::make_integer_sequence<int, kGroups>{}, lds, code[i], F, Ah[i][0], Ah[i][1], sc[i]);
          } else {
            key_groups<float>(std::make_integer_sequence<int, kGroups>{}, lds, code[i], fine, Ah[i], Al[i], sc[i]);
          }
          request_codes(r + 1, i);
        }
      }
    }
  }

  // ------------------------------------------------------------------------------ split softmax
  float m_h[kGqa], l_h[kGqa];
  {
    float mx[kGqa] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      const bool ok = i < my_blocks && (wave + kWaves * i) * 64 + lane < nvalid;
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        sc[i][h] = ok ? sc[i][h] * a.scale : -INFINITY;
        mx[h] = fmaxf(mx[h], sc[i][h]);
      }
    }
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      mx[h] = wave_max(mx[h]);
      if (lane == 0) red[0][wave][h] = mx[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kGqa; ++h)
      m_h[h] = fmaxf(fmaxf(red[0][0][h], red[0][1][h]), fmaxf(red[0][2][h], red[0][3][h]));
    float sm[kGqa] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i)
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        sc[i][h] = __expf(sc[i][h] - m_h[h]);  // masked tokens: exp(-inf) = 0
        sm[h] += sc[i][h];
      }
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      sm[h] = wave_sum(sm[h]);
      if (lane == 0) red[1][wave][h] = sm[h];
    }
    __syncthreads();  // also: every wave is done with the last key table
#pragma unroll
    for (int h = 0; h < kGqa; ++h) l_h[h] = (red[1][0][h] + red[1][1][h]) + (red[1][2][h] + red[1][3][h]);
  }

  // p^T operands: lane 4b+j holds head j's weights for the 4 tokens of its quad (quad transpose)
  const h4 ident = identity_b(lane);
  h4 pth[kMaxBlocks], ptl[kMaxBlocks];
  {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      if constexpr (!kF32) {
        pth[i] = to_h4(mfma(to_h4(sc[i]), ident, z));
        ptl[i] = pth[i];
      } else {
        h4 ph_, pl_;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const Split2 sp = split2(sc[i][e]);
          ph_[e] = sp.hi;
          pl_[e] = sp.lo;
        }
        pth[i] = to_h4(mfma(ph_, ident, z));
        ptl[i] = to_h4(mfma(pl_, ident, z));
      }
    }
  }

  // ------------------------------------------------------------------------------ value phases
  f4 O[2 * kGroups];
#pragma unroll
  for (int c = 0; c < 2 * kGroups; ++c) O[c] = (f4){0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < R; ++r) {
    if (r > 0) __syncthreads();
    load_table<T, R>(cb_v, r, lds, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      if (i < my_blocks) {
        value_groups<T>(std::make_integer_sequence<int, kGroups>{}, lds, code[i], ident, pth[i], ptl[i], O);
        if (r + 1 < R) request_codes(R + r + 1, i);
      }
    }
  }

  // ------------------------------------------------------------------------ workgroup reduction
  // O[c] in lane 16*rho + 4*b' + j, register h: head h, dim 4c + j, summed over the tokens of quad b'.
  // Sum the 4 quads of each 16-lane row with DPP, then the 4 rows and 4 waves through LDS.
  __syncthreads();  // every wave is done with the value table; its space is reused below
  float* red_o = reinterpret_cast<float*>(lds);  // [wave][rho][j][c*4 + h]
#pragma unroll
  for (int c = 0; c < 2 * kGroups; ++c)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      float v = O[c][h];
      v += row_ror<8>(v);
      v += row_ror<4>(v);
      O[c][h] = v;
    }
  if ((lane & 15) < 4) {
    const int rho = lane >> 4, j = lane & 3;
    float* dst = red_o + ((wave * 4 + rho) * 4 + j) * (2 * kGroups * kGqa);
#pragma unroll
    for (int c = 0; c < 2 * kGroups; ++c) *reinterpret_cast<f4*>(dst + c * 4) = O[c];
  }
  __syncthreads();
  const int64_t part_row = static_cast<int64_t>(a.n_splits) * kPartFloats;
  float* part = a.part + ((static_cast<int64_t>(b) * a.n_q_heads + h0) * a.n_splits + split) * kPartFloats;
  // Partials are written with device-scope (agent) atomic stores, which write through to the device
  // coherence point, so no workgroup needs a device-wide release fence (on this chip that fence writes
  // back the whole L2 and costs far more than the stores). Once the stores have completed (vmcnt), the
  // arrival counter is bumped; the last workgroup to arrive merges.
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = tid + kAttnThreads * k;  // (h, d)
    const int h = o >> 7, d = o & 127, c = d >> 2, j = d & 3;
    float acc = 0.f;
#pragma unroll
    for (int wr = 0; wr < 16; ++wr) acc += red_o[(wr * 4 + j) * (2 * kGroups * kGqa) + c * 4 + h];
    __hip_atomic_store(part + h * part_row + 4 + d, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < kGqa) {
    __hip_atomic_store(part + tid * part_row + 0, m_h[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(part + tid * part_row + 1, l_h[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ------------------------------------------------------------------------ last workgroup merges
  const int ns = (L + S - 1) / S;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(a.counters + b * a.n_kv_heads + kv, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == static_cast<uint32_t>(ns - 1));
  }
  __syncthreads();
  if (!is_last) return;
  // Only the merging workgroup pays for an acquire: drop any stale cached copy of the partials.
  __threadfence();
  const float* pb = a.part + (static_cast<int64_t>(b) * a.n_q_heads + h0) * a.n_splits * kPartFloats;
  float* sw = reinterpret_cast<float*>(lds);  // [kGqa][n_splits] split weights e^{m_s - M}
  __shared__ float merge_den[kGqa];
  // one wave per head: max over splits, weights, denominator
  {
    const float* ph = pb + wave * part_row;
    float mx = -INFINITY;
    for (int s2 = lane; s2 < ns; s2 += 64) mx = fmaxf(mx, ph[s2 * kPartFloats]);
    mx = wave_max(mx);
    float den = 0.f;
    for (int s2 = lane; s2 < ns; s2 += 64) {
      const float w = __expf(ph[s2 * kPartFloats] - mx);
      sw[wave * a.n_splits + s2] = w;
      den = fmaf(w, ph[s2 * kPartFloats + 1], den);
    }
    den = wave_sum(den);
    if (lane == 0) merge_den[wave] = den;
  }
  __syncthreads();
  // each thread merges 2 outputs; the split loop issues 16 independent loads per step
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = tid + kAttnThreads * k;
    const int h = o >> 7, d = o & 127;
    const float* ph = pb + h * part_row + 4 + d;
    const float* wh = sw + h * a.n_splits;
    float acc[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc[u] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = s0 + u < ns ? ph[(s0 + u) * kPartFloats] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) acc[u] = fmaf(s0 + u < ns ? wh[s0 + u] : 0.f, v[u], acc[u]);
    }
    float num = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) num += acc[u];
    out_bh[o] = num / merge_den[h];
  }
  if (tid == 0) __hip_atomic_store(a.counters + b * a.n_kv_heads + kv, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_attn(int dtype, int R, int B, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_splits, a.n_kv_heads, B);
  if (dtype == COMMVQ_F16) {
    if (R == 1) attn_kernel<f16, 1><<<grid, kAttnThreads, 0, s>>>(a);
    else attn_kernel<f16, 2><<<grid, kAttnThreads, 0, s>>>(a);
  } else {
    if (R == 1) attn_kernel<float, 1><<<grid, kAttnThreads, 0, s>>>(a);
    else attn_kernel<float, 2><<<grid, kAttnThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace commvq
