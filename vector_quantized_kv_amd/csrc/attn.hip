// Decode-step attention over a CommVQ cache on gfx950, fp32 storage of the byte layout (16 groups x 256
// codes, R = 1 or 2). fp16 storage runs the kernel in attn_f16.hip; launch_attn dispatches both.
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
// Work item: one workgroup of 4 waves per (sequence b, KV head, split of `split_tokens` tokens). Each wave
// owns 64-token blocks; lane = token within the block, so the fine RoPE phase e^{i (t mod 64) theta_j} is
// a per-lane value read from the fp32 table.
//
// Phases K residual 0..R-1, then V residual 0..R-1, each a pass over the split's blocks with that
// residual's codebook (16 groups x 256 codes x 8 floats = 128 KiB) in the one LDS slot, loaded between
// phases by direct global->LDS loads. The code records of the next phase are requested as soon as a block
// has consumed its record of the current one.
//   K phase: gather the token's 16 codeword rows (32 bytes each), rotate them by the fine phase in fp32,
//            and form the 4 GQA head scores with v_mfma_f32_4x4x4_16b_f16 on fp16 hi + lo parts of both
//            operands (hi*hi + hi*lo + lo*hi): B = the token's rotated key (4 dims per step), A = the query
//            rotated by the conjugate coarse phase of the block, broadcast from one 4-lane block
//            (CBSZ/ABID) so each lane supplies only 4 of the 64 query pairs. Scores accumulate across
//            residuals in the MFMA accumulator.
//   softmax: per wave, m_w = max and l_w = sum of p = e^{s - m_w} over the wave's tokens; no barrier.
//   V phase: gather value rows, transpose each 4x4 (token x dim) tile of a lane quad with an identity-B
//            MFMA (exact on fp16 parts), and accumulate p^T x v with three hi/lo products.
// The workgroup then combines its waves (rescaling wave w by e^{m_w - M}), writes (M, L, o[128]) per q
// head, and the last workgroup of each (b, kv) (arrival counter in the workspace, reset to zero by that
// workgroup) merges the splits and writes out.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>
#include <utility>

#include "attn_common.h"

namespace commvq {
namespace {

constexpr int kW32 = 4;                                   // waves per workgroup
constexpr int kTab32 = kGroups * kCodes * kGroupDim * 4;  // one residual's codebook, fp32 (128 KiB)

// Key step for group G of one 64-token block: gather the 8-float row, rotate it by the fine phase in fp32,
// then two MFMA steps (4 dims each) of three hi/lo products.
template <int G>
__device__ __forceinline__ void key_group(const unsigned char* tab, const uint4& code, const float2* fine,
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
  constexpr int m = G < 8 ? 0 : 1;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    h4 bh, bl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const Split2 s = split2(w[4 * st + e]);
      bh[e] = s.hi;
      bl[e] = s.lo;
    }
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

// Value step for group G: gather 8 dims, quad-transpose 2 tiles, accumulate p^T v into O[2G], O[2G+1].
template <int G>
__device__ __forceinline__ void value_group(const unsigned char* tab, const uint4& code, const h4& ident,
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

template <int R>
__global__ void __launch_bounds__(kW32 * 64) attn_f32_kernel(const AttnArgs a) {
  constexpr int kW = kW32;
  constexpr int kThreads = kW * 64;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kTab32];
  __shared__ float wave_ml[2][kW][kGqa];  // per wave and head: softmax max m_w and sum l_w
  __shared__ int is_last;

  // XCD-aware work order: the KV head is the fastest grid index. Workgroups are dealt to the 8 XCDs in
  // turn, so with 8 KV heads each XCD serves one head and its L2 fetches only that head's codebooks.
  const int kv = blockIdx.x % a.n_kv_heads, split = blockIdx.x / a.n_kv_heads, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave values scalar
  const int64_t cb_stride = static_cast<int64_t>(kGroups) * R * kCodes * kGroupDim;
  const float* cb_k = static_cast<const float*>(a.k_cb) + kv * cb_stride;
  const float* cb_v = static_cast<const float*>(a.v_cb) + kv * cb_stride;
  auto table_src = [&](int p) { return p < R ? cb_k : cb_v; };
  // sequence bounds (clamped), read before any memory operation so that they stay scalar loads
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.max_len, a.total_tokens);
  const int L = sb.len;
  const int64_t seq_start = sb.start;

  // ---------------------------------------------------------------------------------- prologue
  // (1) The first key codebook, straight into LDS. It depends on nothing but the KV head, so it goes out
  // before the sequence bounds have arrived.
  load_table<float, R, kW>(cb_k, 0, lds, wave, lane);
  __builtin_amdgcn_sched_barrier(0);

  const int S = a.split_tokens;
  const int t0 = split * S;
  const int h0 = kv * kGqa;
  const int64_t bh0 = static_cast<int64_t>(b) * a.n_q_heads + h0;
  float* out_bh = a.out + bh0 * kHeadDim;
  if (t0 >= L) {
    if (split == 0)  // empty sequence: the output is zero
      for (int i = tid; i < kGqa * kHeadDim; i += kThreads) out_bh[i] = 0.f;
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));  // the direct-to-LDS loads land before the workgroup ends
    return;
  }
  const int nvalid = min(S, L - t0);
  const int nblocks = (nvalid + 63) >> 6;
  const int my_blocks = (nblocks - wave + kW - 1) / kW;  // this wave owns blocks wave, wave + kW, ...
  const int64_t row_base = seq_start + t0;

  // token row of block i for this lane, clamped into the split so every load is in bounds
  auto token_row = [&](int i) -> int64_t {
    int tl = (wave + kW * i) * 64 + lane;
    asm volatile("" : "+v"(tl));  // recomputed at every use: 8 blocks' row offsets kept live would take 16 VGPRs
    return row_base + min(tl, nvalid - 1);
  };

  // (2) register operands: query pairs and the coarse phases of every block.
  // Query pairs this lane supplies to the broadcast A operand: head qi, pairs 2*quad + {0,1} (+32).
  const int quad = lane >> 2, qi = lane & 3;
  const float* qp = static_cast<const float*>(a.q) + (bh0 + qi) * kHeadDim;
  // index 2m + e is pair 32m + 2 quad + e
  float2 qv[4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) qv[2 * m + e] = *reinterpret_cast<const float2*>(qp + 2 * (32 * m + 2 * quad + e));
  const float2* coarse = a.rope + kRopeCoarseOffset;
  // coarse phases of this lane's 4 query pairs for every block (rows clamped to the split's last block,
  // so always inside the table)
  float4 cphase[kMaxBlocks][2];
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) {
    const float2* cr = coarse + static_cast<int64_t>((t0 >> 6) + min(wave + kW * i, nblocks - 1)) * kPairs;
#pragma unroll
    for (int m = 0; m < 2; ++m) cphase[i][m] = *reinterpret_cast<const float4*>(cr + 32 * m + 2 * quad);
  }
  const float2* fine = a.rope + lane;  // fine[j * 64 + lane], read per group
  __builtin_amdgcn_sched_barrier(0);
  // (3) code records of phase 0. Code records of the current phase live in code[]; once a block has
  // consumed its record, the record of the same token for the next phase is requested.
  uint4 code[kMaxBlocks];
  auto request_codes = [&](int ph, int i) {
    const uint8_t* base = ph < R ? a.k_codes : a.v_codes;
    code[i] = load_code_record(base, a.total_tokens, kv, token_row(i), R, ph % R);
  };
  // The prologue requests the records of the first kLeadBlocks blocks only (a wave's full share would
  // queue a large part of the whole code stream ahead of the codebook loads); block i of the first phase
  // requests block i + kLeadBlocks.
  constexpr int kLeadBlocks = kMaxBlocks < 3 ? kMaxBlocks : 3;
#pragma unroll
  for (int i = 0; i < kLeadBlocks; ++i) request_codes(0, i);

  // End of phase p: every wave is done with the slot; load the codebook of phase p + 1 into it.
  auto next_phase = [&](int p) {
    slot_barrier();
    load_table<float, R, kW>(table_src(p + 1), (p + 1) % R, lds, wave, lane);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    slot_barrier();
  };
  // The first codebook was issued before the code records, which the barrier keeps last. Nothing may
  // wait on a loaded register between the codebook loads and this point: while a direct-to-LDS load is
  // outstanding the compiler can only wait with vmcnt(0), which would include the records.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kLeadBlocks));
  slot_barrier();
  // Pin the query and coarse-phase registers here, so the arithmetic on them (and its wait for their
  // loads) cannot be hoisted above the codebook loads.
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(qv[k].x), "+v"(qv[k].y));
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
      asm volatile("" : "+v"(cphase[i][m].x), "+v"(cphase[i][m].y), "+v"(cphase[i][m].z), "+v"(cphase[i][m].w));

  // A operands: the query rotated by the conjugate coarse phase of each 64-token block, q'' = q * conj(C),
  // as fp16 hi and lo parts; the same for every key phase.
  h4 Ah[kMaxBlocks][2], Al[kMaxBlocks][2];
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float4 c = cphase[i][m];
      const float2 u0 = cmul_conj(qv[2 * m], make_float2(c.x, c.y));
      const float2 u1 = cmul_conj(qv[2 * m + 1], make_float2(c.z, c.w));
      const float qq[4] = {u0.x, u0.y, u1.x, u1.y};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const Split2 sp = split2(qq[e]);
        Ah[i][m][e] = sp.hi;
        Al[i][m][e] = sp.lo;
      }
    }
  }

  // ------------------------------------------------------------------------------ key phases
  f4 sc[kMaxBlocks];
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) sc[i] = (f4){0.f, 0.f, 0.f, 0.f};
  // Residual phases are instantiated with compile-time r (straight-line code), so that every wait for a
  // prefetched record is an exact vmcnt rather than a conservative one at a loop header.
  auto key_phase = [&](auto rc) {
    constexpr int r = decltype(rc)::value;
    static_for<kMaxBlocks>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (r == 0 && i + kLeadBlocks < kMaxBlocks) request_codes(0, i + kLeadBlocks);
      if (i < my_blocks)
        static_for<kGroups>([&](auto gc) { key_group<decltype(gc)::value>(lds, code[i], fine, Ah[i], Al[i], sc[i]); });
      request_codes(r + 1, i);  // phase r + 1 always exists (the value phases follow)
    });
    if constexpr (r + 1 < R) next_phase(r);
  };
  key_phase(std::integral_constant<int, 0>{});
  if constexpr (R > 1) key_phase(std::integral_constant<int, 1>{});

  // ------------------------------------------------------------------------------ wave softmax
  wave_softmax<kW>(sc, my_blocks, wave, lane, nvalid, a.scale, wave_ml);

  // p^T operands: lane 4b+j holds head j's weights for the 4 tokens of its quad (quad transpose), as fp16
  // hi and lo parts
  const h4 ident = identity_b(lane);
  h4 pth[kMaxBlocks], ptl[kMaxBlocks];
  {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
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
  next_phase(R - 1);  // the first value codebook

  // ------------------------------------------------------------------------------ value phases
  f4 O[2 * kGroups];
#pragma unroll
  for (int c = 0; c < 2 * kGroups; ++c) O[c] = (f4){0.f, 0.f, 0.f, 0.f};
  auto value_phase = [&](auto rc) {
    constexpr int r = decltype(rc)::value;
    constexpr int p = R + r;
    static_for<kMaxBlocks>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (i < my_blocks)
        static_for<kGroups>([&](auto gc) { value_group<decltype(gc)::value>(lds, code[i], ident, pth[i], ptl[i], O); });
      if constexpr (r + 1 < R) request_codes(p + 1, i);
    });
    if constexpr (r + 1 < R) next_phase(p);
  };
  value_phase(std::integral_constant<int, 0>{});
  if constexpr (R > 1) value_phase(std::integral_constant<int, 1>{});

  // ------------------------------------------------------------------------ workgroup reduction
  // (Lane and thread indices are recomputed here so that no index register lives across the phases.)
  attn_epilogue<kW>(a, lds, wave_ml, is_last, lane_id(), wave * 64 + lane_id(), wave, O, b, kv, split, L, S, bh0,
                    out_bh);
}

}  // namespace

hipError_t launch_attn(int dtype, int R, int B, const AttnArgs& a, hipStream_t s) {
  if (dtype == COMMVQ_F16) return launch_attn_f16(R, B, a, s);
  dim3 grid(a.n_splits * a.n_kv_heads, B);
  if (R == 1) attn_f32_kernel<1><<<grid, kW32 * 64, 0, s>>>(a);
  else attn_f32_kernel<2><<<grid, kW32 * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace commvq
