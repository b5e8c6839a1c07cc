// Device pieces shared by the attention kernels (byte layout in fp16 and fp32 storage, bit-packed records):
// fp16 vector types, MFMA wrappers, workgroup barriers, codebook staging, the wave softmax and the epilogue
// (workgroup combine of the waves' partial outputs, split partials, last-workgroup merge).
#pragma once

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

constexpr int kMaxBlocks = kAttnMaxBlocksPerWave;

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave are outstanding
// (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_at_most(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

template <int ABID>
__device__ __forceinline__ f4 mfma_bcast(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}
__device__ __forceinline__ f4 mfma(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0); }

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ h4 cat(h2 a, h2 b) { return (h4){a.x, a.y, b.x, b.y}; }
__device__ __forceinline__ h4 to_h4(f4 x) { return (h4){(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]}; }

struct Split2 {  // fp32 value as fp16 hi + lo
  f16 hi, lo;
};
__device__ __forceinline__ Split2 split2(float x) {
  f16 h = (f16)x;
  return {h, (f16)(x - (float)h)};
}

// s_waitcnt immediate that waits for all of this wave's LDS operations (lgkmcnt = 0) and nothing else.
constexpr int kLgkmcnt0 = 0xf | (0x3 << 14) | (0x7 << 4);

// Workgroup barriers that leave this wave's global loads in flight. __syncthreads() releases memory at
// workgroup scope, which on this target waits for every outstanding vector-memory load of the wave,
// including code records prefetched for later blocks (and a release that only covers LDS still waits
// for them while a direct-to-LDS load is pending).
// lds_barrier: LDS writes before it are visible to every wave after it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// slot_barrier: codebook slot hand-over. Each wave has already waited (vmcnt) for its own direct-to-LDS
// loads into the slot being published; lgkmcnt(0) retires this wave's reads of the slot about to be
// refilled. Nothing is written to LDS by ordinary stores across it, so no release is needed.
__device__ __forceinline__ void slot_barrier() {
  __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// This lane's index in its wave, computed afresh rather than kept in a register since the kernel began.
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Transposing LDS read (ds_read_b64_tr_b16): every lane names 8 bytes (4 fp16 values) of LDS; within each
// 16-lane group, lane 4a + e receives value e of the loads named by lanes a, a + 4, a + 8 and a + 12 (in
// that order). For MFMA block b = 4g + a of the 4x4x4 instruction, that is a 4x4 transpose: B_b[k][e]
// is value e of source lane 16g + 4k + a.
__device__ __forceinline__ h4 lds_read_tr(const void* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p)));
}

// Identity B operand: lane 4b+j holds e_j, so D_b = A_b (a quad transpose of A).
__device__ __forceinline__ h4 identity_b(int lane) {
  const int j = lane & 3;
  return (h4){(f16)(j == 0), (f16)(j == 1), (f16)(j == 2), (f16)(j == 3)};
}

// fp16 block loops are software pipelines over units (a quarter or a pair of groups): the gathers of unit
// n + kAhead go out before the arithmetic of unit n, rotating through kAhead + 1 register buffers.
constexpr int kAhead = 2;
constexpr int kBufs = kAhead + 1;
// Wave priority while a wave works on block i of a phase: higher for waves with more blocks left, so the
// two waves that share a SIMD advance together instead of the older one finishing first.
constexpr int block_prio(int i) { return (kAttnMaxBlocksPerWave - 1 - i) * 3 / (kAttnMaxBlocksPerWave - 1); }

__device__ __forceinline__ uint32_t add_h2(uint32_t x, uint32_t y) { return __builtin_bit_cast(uint32_t, as_h2(x) + as_h2(y)); }
__device__ __forceinline__ uint4 add_rows(const uint4& x, const uint4& y) {
  return make_uint4(add_h2(x.x, y.x), add_h2(x.y, y.y), add_h2(x.z, y.z), add_h2(x.w, y.w));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time unrolled).
template <int... Is, typename Fn>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, Fn&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

inline __device__ float2 cmul_conj(float2 x, float2 c) { return make_float2(x.x * c.x + x.y * c.y, x.y * c.x - x.x * c.y); }

// Fill one codebook slot (16 groups x 256 codes, row = 8 values of T) with direct global->LDS 16-byte
// loads; each wave moves its share. cb_kv points at codebook [kv][0][0][0][0]; r selects the residual.
template <typename T, int R, int kW>
__device__ __forceinline__ void load_table(const T* cb_kv, int r, unsigned char* dst, int wave, int lane) {
  constexpr int kRowBytes = kGroupDim * sizeof(T);
  constexpr int kChunksPerRow = kRowBytes / 16;
  constexpr int kChunks = kGroups * kCodes * kChunksPerRow;
  constexpr int kPerWave = kChunks / kW;
#pragma unroll
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

// Wave softmax over the wave's blocks (block i holds tokens (wave + kW i) * 64 + lane of the split): scales
// the scores, masks tokens at or past nvalid, overwrites them with p, and returns (m_w, l_w) per head
// (wave-uniform values).
template <int kW>
__device__ __forceinline__ void wave_softmax_regs(f4 (&sc)[kMaxBlocks], const int my_blocks, const int wave,
                                                  const int lane, const int nvalid, const float scale,
                                                  float (&m_w)[kGqa], float (&l_w)[kGqa]) {
  // m_w = max over the wave's valid tokens, p = e^{s - m_w}, l_w = sum p. A wave with no valid token
  // has m_w = -inf, p = 0, l_w = 0, and weight e^{m_w - M} = 0 in the workgroup combine.
#pragma unroll
  for (int h = 0; h < kGqa; ++h) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      const bool ok = i < my_blocks && (wave + kW * i) * 64 + lane < nvalid;
      sc[i][h] = ok ? sc[i][h] * scale : -INFINITY;
      mx = fmaxf(mx, sc[i][h]);
    }
    m_w[h] = wave_max(mx);
    const float msafe = m_w[h] == -INFINITY ? 0.f : m_w[h];
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      sc[i][h] = __expf(sc[i][h] - msafe);  // masked tokens: exp(-inf) = 0
      sm += sc[i][h];
    }
    l_w[h] = wave_sum(sm);
  }
}
// The same, publishing (m_w, l_w) in LDS for the workgroup epilogue.
template <int kW>
__device__ __forceinline__ void wave_softmax(f4 (&sc)[kMaxBlocks], const int my_blocks, const int wave, const int lane,
                                             const int nvalid, const float scale, float (&wave_ml)[2][kW][kGqa]) {
  float m_w[kGqa], l_w[kGqa];
  wave_softmax_regs<kW>(sc, my_blocks, wave, lane, nvalid, scale, m_w, l_w);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      wave_ml[0][wave][h] = m_w[h];
      wave_ml[1][wave][h] = l_w[h];
    }
  }
}

// Workgroup epilogue of a decode-attention work item (one split of one (sequence, KV head)): O holds this
// wave's unnormalised p^T v in the quad layout of the value MFMAs, wave_ml every wave's (m_w, l_w).
// With ml_regs set, (m_w, l_w) arrive in registers (wave_ml and is_last then point into the codebook space, past
// the reduction buffer) and are published once every wave is done with the codebooks.
template <int kW>
__device__ __forceinline__ void attn_epilogue(const AttnArgs& a, unsigned char* lds, float (&wave_ml)[2][kW][kGqa],
                                              int& is_last, const int lane, const int tid, const int wave,
                                              f4 (&O)[2 * kGroups], const int b, const int kv, const int split,
                                              const int L, const int S, const int64_t bh0, float* out_bh,
                                              const float* ml_regs_m = nullptr, const float* ml_regs_l = nullptr) {
  constexpr int kThreads = kW * 64;
  lds_barrier();  // every wave is done with the value codebooks; their space is reused below
  if (ml_regs_m != nullptr && lane == 0) {
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      wave_ml[0][wave][h] = ml_regs_m[h];
      wave_ml[1][wave][h] = ml_regs_l[h];
    }
  }

  // O[c][h] sits in lane 16*rho + 4*b' + j (head h, dim 4c + j, one token quad per (rho, b')); each output
  // is the sum over the 16 lanes that share j. Two half-wave swap steps first fold the rows: each step pairs
  // two registers and halves the register count, so for every q the four rows of W[q] end up holding dims
  // 4c + j of c = 4q + rho, each summed over its 4 rows. DPP then sums the 4 quads of every row.
  float W[2 * kGroups / 4][kGqa];
#pragma unroll
  for (int q = 0; q < 2 * kGroups / 4; ++q)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      const float z0 = swap32_add(O[4 * q][h], O[4 * q + 2][h]);      // rows 0,1: c = 4q;     rows 2,3: c = 4q + 2
      const float z1 = swap32_add(O[4 * q + 1][h], O[4 * q + 3][h]);  // rows 0,1: c = 4q + 1; rows 2,3: c = 4q + 3
      W[q][h] = swap16_add(z0, z1);                                    // row rho: c = 4q + rho
    }
#pragma unroll
  for (int q = 0; q < 2 * kGroups / 4; ++q)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) W[q][h] += row_ror<8>(W[q][h]);
#pragma unroll
  for (int q = 0; q < 2 * kGroups / 4; ++q)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      W[q][h] += row_ror<4>(W[q][h]);
      asm("" : "+v"(W[q][h]));  // keeps the add beside its DPP move (one v_add_f32_dpp), not in the store branch
    }
  // red_o [wave][d][h]: lanes 16*rho + j (j < 4) store dims d = 16q + 4rho + j, so each store instruction
  // covers 256 contiguous bytes; the readers (one (h, d) each) walk consecutive entries.
  float* red_o = reinterpret_cast<float*>(lds);
  if ((lane & 15) < 4) {
    const int rho = lane >> 4, j = lane & 3;
    f4* dst = reinterpret_cast<f4*>(red_o) + wave * kHeadDim + 4 * rho + j;
#pragma unroll
    for (int q = 0; q < 2 * kGroups / 4; ++q) dst[16 * q] = (f4){W[q][0], W[q][1], W[q][2], W[q][3]};
  }
  lds_barrier();
  // Partials are written with device-scope (agent) atomic stores, which write through to the device
  // coherence point, so no workgroup needs a device-wide release fence (on this chip that fence writes
  // back the whole L2 and costs far more than the stores). Once the stores have completed (vmcnt), the
  // arrival counter is bumped; the last workgroup to arrive merges.
  const int64_t ns_alloc = a.n_splits;
#pragma unroll
  for (int k = 0; k < kGqa * kHeadDim / kThreads; ++k) {
    const int o = tid + kThreads * k;  // (h, d)
    const int h = o >> 7, d = o & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, wave_ml[0][w][h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float f = __expf(wave_ml[0][w][h] - M);  // 0 for a wave without tokens
      acc = fmaf(f, red_o[(w * kHeadDim + d) * kGqa + h], acc);
      lsum = fmaf(f, wave_ml[1][w][h], lsum);
    }
    const int64_t item = (bh0 + h) * ns_alloc + split;
    __hip_atomic_store(a.part_o + item * kHeadDim + d, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      float* ml = reinterpret_cast<float*>(a.part_ml + item);
      __hip_atomic_store(ml, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ml + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
  // The partials are read with device-scope (agent) loads, which read through to the coherence point the
  // partial stores wrote through to; this replaces an acquire fence, which on this chip invalidates the
  // whole L2.
  // Per chunk of up to kChunk splits, one memory round trip: the first kGqa * kChunk threads each load one
  // (m_s, l_s) into LDS (the reduction buffer, free again), and every thread loads the partial o_s[d] of its
  // output (h, d) for every split of the chunk; after the barrier each thread combines its output, a running
  // maximum rescaling earlier chunks (one chunk covers 32 splits: 128K tokens at the largest split).
  constexpr int kChunk = 32;
  constexpr int kOut = kGqa * kHeadDim / kThreads;
  static_assert(kGqa * kChunk <= kThreads, "one (m, l) load per thread");
  float2* ml_lds = reinterpret_cast<float2*>(lds);
  float M[kOut], num[kOut], den[kOut];
#pragma unroll
  for (int k = 0; k < kOut; ++k) {
    M[k] = -INFINITY;
    num[k] = 0.f;
    den[k] = 0.f;
  }
  for (int s0 = 0; s0 < ns; s0 += kChunk) {
    if (s0 > 0) __syncthreads();  // every thread is done with the previous chunk's (m, l)
    if (tid < kGqa * kChunk) {
      const int h = tid / kChunk, u = tid % kChunk;
      const float* pm = reinterpret_cast<const float*>(a.part_ml + (bh0 + h) * ns_alloc + s0 + u);
      ml_lds[tid] = s0 + u < ns ? make_float2(__hip_atomic_load(pm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                              __hip_atomic_load(pm + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                                : make_float2(-INFINITY, 0.f);
    }
    float v[kOut][kChunk];
#pragma unroll
    for (int k = 0; k < kOut; ++k) {
      const int o = tid + kThreads * k;
      const int h = o >> 7, d = o & 127;
      const float* po = a.part_o + ((bh0 + h) * ns_alloc + s0) * kHeadDim + d;
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        v[k][u] = s0 + u < ns ? __hip_atomic_load(po + static_cast<int64_t>(u) * kHeadDim, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : 0.f;
    }
    __syncthreads();  // the chunk's (m, l) are in LDS
#pragma unroll
    for (int k = 0; k < kOut; ++k) {
      const int h = (tid + kThreads * k) >> 7;
      const float2* ml = ml_lds + h * kChunk;
      float mc = M[k];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) mc = fmaxf(mc, ml[u].x);  // finite: split 0 always has tokens
      const float r = __expf(M[k] - mc);  // 0 on the first chunk
      num[k] *= r;
      den[k] *= r;
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const float w = __expf(ml[u].x - mc);  // 0 past the last split
        num[k] = fmaf(w, v[k][u], num[k]);
        den[k] = fmaf(w, ml[u].y, den[k]);
      }
      M[k] = mc;
    }
  }
#pragma unroll
  for (int k = 0; k < kOut; ++k) out_bh[tid + kThreads * k] = num[k] / den[k];
  if (tid == 0) __hip_atomic_store(a.counters + b * a.n_kv_heads + kv, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace commvq
