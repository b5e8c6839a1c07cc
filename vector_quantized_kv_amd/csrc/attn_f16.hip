// Decode-step attention over a CommVQ cache with fp16 codebooks (byte layout: one index byte per group,
// 16 groups of 8 dims, N = 256, R = 1 or 2) on gfx950: one fused kernel per call.
//
// What it computes (sources by page title and section):
//   score_t = scale * sum_j Re( conj(q_j) * khat_{t,j} * e^{i t theta_j} )
//   out     = sum_t softmax(score)_t * vhat_t
// with khat, vhat the additive decodes (sum over R residual codebooks) of the stored code indices
// ("1-bit quantization" tag page, CommVQ abstract; pith.science verdict for arXiv 2506.18879,
// pith_extraction.key_machinery). Each key codeword block [[a,-b],[b,a]] commutes with the RoPE rotation,
// so the rotation by position splits freely between the query and the key side: the part shared by a
// 64-token block (e^{i 64 c theta}) goes on the query once per block, the per-token part e^{i f theta},
// f = t mod 64 = lane, on the gathered codeword.
//
// Work item: one workgroup per (sequence b, KV head, split of `split_tokens` tokens), one per CU (it owns
// the CU's LDS); 8 waves, each owning 64-token blocks (lane = token), up to 8 blocks per wave.
//
// Key scores are formed in fp32: the per-token rotation of the (residual-summed) codeword is computed in
// fp32 from fp32 phases and contracted with the fp32 block query on the fp32 matrix core
// (v_mfma_f32_4x4x1_16b_f32, query broadcast from one 4-lane block per dim). On this chip the fp32 MFMA does
// not run beside VALU work of the SIMD (the fp16 ones do), and alternating the two costs extra cycles, so
// the rotations and the MFMAs of a group are issued as separate bursts. fp16 operands would round the
// key and the query to 11 bits, which at realistic logit ranges (score spreads of 10 and more) moves the
// softmax by more than the 2e-3 output tolerance; in fp32 the key path is exact to a few fp32 ulps.
// The fp32 phases of one lane (64 pairs) would take 128 registers, so they stay in LDS (32 KiB) and the key
// pass runs group-major: a wave reads one group's phases once and applies them to 2 of its blocks (one
// "sweep"); a wave with an even number of blocks makes one sweep per two, a wave with an odd number goes block
// by block.
//
// LDS: two residual codebooks (64 KiB each: 16 groups x 256 rows x 8 fp16) and the phase table (32 KiB) fill
// the CU's 160 KiB (map below). R = 1: key and value codebook, both loaded in the prologue. R = 2: the two key
// codebooks, replaced by the two value codebooks in two halves (groups 0-7, then 8-15) as the passes move on.
//
// Value pass (fp16 operands, fp32 accumulation; the softmax weights and value codewords are rounded
// to fp16 once): each group's rows are gathered whole (R = 2: both residuals, summed in fp16), each 4x4
// (token x dim) tile of a lane quad is transposed with an identity MFMA, and p^T x v accumulates with the
// 4x4x4 MFMA.
// The workgroup combines its waves, writes (M, L, o[128]) per q head, and the last workgroup of each
// (b, kv) merges the splits (attn_common.h).
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>
#include <utility>

#include "attn_common.h"

namespace commvq {
namespace {

constexpr int kW16 = 8;                              // waves per workgroup
constexpr int kThreads16 = kW16 * 64;

constexpr int kPhaseBytes = kGroups * 2 * 64 * 16;  // fp32 fine phases [g][h][lane][2 pairs]
constexpr int kSweep = 2;                            // blocks per key sweep
constexpr int kValueLead = 4;                        // value records requested this many blocks ahead

// fp32 4x4x1 MFMA with the A operand broadcast from block ABID: acc[m] += A[lane 4 ABID + m] * b.
template <int ABID>
__device__ __forceinline__ f4 mfma32_bcast(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 4, ABID, 0);
}

// Rotated key of one group: the lane's gathered row(s) (4 pairs (a, b) in fp16), summed over residuals in fp32,
// times the lane's fine phases (p0 = pairs 4G, 4G+1, p1 = 4G+2, 4G+3, each (cos, sin)) in fp32:
// w[2u] + i w[2u+1] = e^{i f theta_j} khat_j for pair j = 4G + u.
// R = 1 reads the fp16 codeword directly (v_fma_mix). R = 2 takes the residual sum from sum_rows (ksum: the
// fp32 entries (a, b, a, b) of pairs 4G, 4G+1 and of 4G+2, 4G+3).
__device__ __forceinline__ void rotate_f32(const f4 (&ksum)[2], const float4& p0, const float4& p1, float (&w)[8]) {
  const float cs[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float c = cs[2 * u], s = cs[2 * u + 1];
    const float kr = ksum[u >> 1][2 * (u & 1)], ki = ksum[u >> 1][2 * (u & 1) + 1];
    w[2 * u] = fmaf(kr, c, -(ki * s));
    w[2 * u + 1] = fmaf(ki, c, kr * s);
  }
}
__device__ __forceinline__ void rotate_f16(const uint4& r0, const float4& p0, const float4& p1, float (&w)[8]) {
  const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
  const float cs[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float c = cs[2 * u], s = cs[2 * u + 1];
    const h2 k = as_h2(w0[u]);  // fp16 operands read directly by v_fma_mix: no conversions
    w[2 * u] = fmaf(static_cast<float>(k.x), c, -fmaf(static_cast<float>(k.y), s, 0.f));
    w[2 * u + 1] = fmaf(static_cast<float>(k.y), c, fmaf(static_cast<float>(k.x), s, 0.f));
  }
}
// Exact fp32 sum of two fp16 rows (R = 2) on the matrix core: with the identity as A, the 4x4x4 MFMA returns in
// each lane its own 4 B values; accumulating the second residual's row adds it in fp32 (one rounding). fp16
// MFMAs run beside the VALU rotations.
__device__ __forceinline__ void sum_rows(const uint4& r0, const uint4& r1, const h4& ident, f4 (&ksum)[2]) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  ksum[0] = mfma(ident, cat(as_h2(r1.x), as_h2(r1.y)), mfma(ident, cat(as_h2(r0.x), as_h2(r0.y)), z));
  ksum[1] = mfma(ident, cat(as_h2(r1.z), as_h2(r1.w)), mfma(ident, cat(as_h2(r0.z), as_h2(r0.w)), z));
}
template <int R>
__device__ __forceinline__ void rotate_key(const uint4& r0, const uint4& r1, const float4& p0, const float4& p1,
                                           const h4& ident, float (&w)[8]) {
  if constexpr (R == 1) {
    rotate_f16(r0, p0, p1, w);
  } else {
    f4 ksum[2];
    sum_rows(r0, r1, ident, ksum);
    rotate_f32(ksum, p0, p1, w);
  }
}
// Contraction of NB blocks' rotated keys of group G with their block queries: per pair j = 4G + u,
// q''_re x w_re + q''_im x w_im, the query of pair j broadcast from block j mod 16 (the lanes holding pair
// 16 (G / 4) + lane / 4). Each block accumulates into two chains (acc[2 i] for the real parts, acc[2 i + 1] for
// the imaginary ones), so consecutive MFMAs never depend on each other.
template <int G, int NB>
__device__ __forceinline__ void contract_key(const float (&w)[NB][8], const float2 (&A)[NB], f4 (&acc)[2 * NB]) {
  static_for<8>([&](auto dc) {
    constexpr int d = decltype(dc)::value;
    constexpr int abid = (4 * G + d / 2) & 15;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      acc[2 * i + (d & 1)] = mfma32_bcast<abid>((d & 1) ? A[i].y : A[i].x, w[i][d], acc[2 * i + (d & 1)]);
  });
}

// Value path: each group's row (R = 2: the fp16 sum of its two residual rows) is gathered whole by the value pass
// from the LDS map below; an identity MFMA transposes each 4-dim half within its lane quad (lane 4b + j receives
// dim j of the quad's 4 tokens, exactly, in fp32), which converted back is the B operand of p^T x v for MFMA
// block b = the quad.
template <int G>
__device__ __forceinline__ void value_step_quad(const uint4& row, const h4& ident, const h4& pt,
                                                f4 (&O)[2 * kGroups]) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  const f4 x0 = mfma(cat(as_h2(row.x), as_h2(row.y)), ident, z);
  const f4 x1 = mfma(cat(as_h2(row.z), as_h2(row.w)), ident, z);
  O[2 * G] = mfma(pt, to_h4(x0), O[2 * G]);
  O[2 * G + 1] = mfma(pt, to_h4(x1), O[2 * G + 1]);
}
template <int P>
__device__ __forceinline__ void value_pair2(const uint4 (&buf)[2][2], const h4& ident, const h4& pt,
                                            f4 (&O)[2 * kGroups]) {
  value_step_quad<2 * P>(add_rows(buf[0][0], buf[0][1]), ident, pt, O);
  value_step_quad<2 * P + 1>(add_rows(buf[1][0], buf[1][1]), ident, pt, O);
}

// LDS map (bytes). Codebook rows are 16 bytes (8 fp16), 4 KiB per (residual, group).
//   R = 2: region A [0, 64 KiB) holds groups 0-7 of both residuals (residual r at r x 32 KiB), the fp32 phases
//          [64, 96 KiB), region B [96, 160 KiB) groups 8-15 (residual r at 96 KiB + r x 32 KiB). The key codebooks
//          are replaced by the value codebooks half by half: region A once every wave is past group 7 of its last
//          key unit, region B once the key pass is over.
//   R = 1: key codebook [0, 64 KiB), phases [64, 96 KiB), value codebook [96, 160 KiB).
// Offsets below 64 KiB go into the LDS instructions' offset field; region B and the R = 1 value codebook are
// addressed from one base register (kHiBase), so a row address costs one or two VALU operations.
constexpr int kKiB = 1024;
// Staged (R = 2): the key pass starts once groups 0-7 have landed and the codebooks are swapped half by half
// as above. Unstaged (R = 1): the prologue waits for every codebook. (Timed per launch on MI355X: staging saves
// about 0.3 us at 8K tokens and is even at 128K for R = 2; for R = 1, whose value codebook is loaded up front
// anyway, the extra barrier in the first key unit costs about 0.5 us at 128K.)
template <int R>
constexpr bool kStagedTables = R == 2;
constexpr int kPhaseOff = 64 * kKiB;
constexpr int kHiBase = 96 * kKiB;
static_assert(kHiBase + 64 * kKiB <= 160 * kKiB, "codebooks and phases fit the CU's LDS");
template <int R>
constexpr int key_row_off(int r, int g) {
  return R == 2 ? (g < 8 ? 0 : kHiBase) + r * 32 * kKiB + (g & 7) * 4 * kKiB : g * 4 * kKiB;
}
template <int R>
constexpr int value_row_off(int r, int g) {
  return R == 2 ? key_row_off<2>(r, g) : kHiBase + g * 4 * kKiB;
}

// Row idx of the table at LDS offset kOff (hi = kHiBase, held in a register).
template <int kOff>
__device__ __forceinline__ uint4 lds_row(const unsigned char* lds, int hi, uint32_t idx) {
  if constexpr (kOff < kHiBase) {
    return *reinterpret_cast<const uint4*>(lds + kOff + idx * 16);
  } else {
    return *reinterpret_cast<const uint4*>(lds + hi + (kOff - kHiBase) + idx * 16);
  }
}

// Direct global->LDS copy of groups g0 .. g0 + kN - 1 of residual r's codebook [G][R][N][8] into LDS at dst
// (4 KiB per group); the copy is cut into kW16 parts and each wave moves part `part` (a permutation of the
// waves, so that the workgroups of one XCD, which all copy the same KV head's codebook at the same moment,
// start on different parts of it and spread their requests over the L2 channels).
template <int R, int kN>
__device__ __forceinline__ void load_groups(const f16* cb_kv, int r, int g0, unsigned char* dst, int part, int lane) {
  constexpr int kPerWave = kN * kCodes / kW16;
#pragma unroll
  for (int i = 0; i < kPerWave / 64; ++i) {
    const int c = part * kPerWave + i * 64 + lane, g = g0 + (c >> 8), l = c & (kCodes - 1);
    const f16* src = cb_kv + ((static_cast<int64_t>(g) * R + r) * kCodes + l) * kGroupDim;
    __builtin_amdgcn_global_load_lds(src, dst + (part * kPerWave + i * 64) * 16, 16, 0, 0);
  }
}

template <int R>
__global__ void __launch_bounds__(kThreads16) attn_f16_kernel(const AttnArgs a) {
  constexpr int kW = kW16;
  __shared__ __attribute__((aligned(16))) unsigned char lds[160 * kKiB];
  // epilogue-only LDS (in region A, past the reduction buffer, once the passes are done)
  auto& wave_ml = *reinterpret_cast<float(*)[2][kW][kGqa]>(lds + kW * kHeadDim * kGqa * sizeof(float));
  int& is_last = *reinterpret_cast<int*>(lds + kW * kHeadDim * kGqa * sizeof(float) + sizeof(wave_ml));

  // XCD-aware work order: the KV head is the fastest grid index. Workgroups are dealt to the 8 XCDs in
  // turn, so with 8 KV heads each XCD serves one head and its L2 fetches only that head's codebooks.
  const int kv = blockIdx.x % a.n_kv_heads, split = blockIdx.x / a.n_kv_heads, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the part of each codebook copy this wave moves: rotated by the split (see load_groups)
  const int part = __builtin_amdgcn_readfirstlane((wave + split) & (kW16 - 1));
  const int64_t cb_stride = static_cast<int64_t>(kGroups) * R * kCodes * kGroupDim;
  const f16* cb_k = static_cast<const f16*>(a.k_cb) + kv * cb_stride;
  const f16* cb_v = static_cast<const f16*>(a.v_cb) + kv * cb_stride;
  // sequence bounds (clamped), read before any memory operation so that they stay scalar loads
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.max_len, a.total_tokens);
  const int L = sb.len;
  const int64_t seq_start = sb.start;

  // ---------------------------------------------------------------------------------- prologue
  // A split past the end of its sequence (a ragged batch launches the longest sequence's split count for every
  // sequence) leaves at once, before any LDS copy: only the record loads, which need the sequence bounds
  // anyway, are on the critical path of the prologue, so testing first costs the other workgroups nothing.
  const int S = a.split_tokens;
  const int t0 = split * S;
  const int h0 = kv * kGqa;
  const int64_t bh0 = static_cast<int64_t>(b) * a.n_q_heads + h0;
  float* out_bh = a.out + bh0 * kHeadDim;
  if (t0 >= L) {
    if (split == 0)  // empty sequence: the output is zero
      for (int i = tid; i < kGqa * kHeadDim; i += kThreads16) out_bh[i] = 0.f;
    return;
  }
  // (1) The key codebook rows of groups 0-7 and the fp32 fine phases, straight into LDS. Groups 8-15 (and the
  // R = 1 value codebook) follow the first records and land while the first key unit works on groups 0-7.
  load_groups<R, 8>(cb_k, 0, 0, lds + key_row_off<R>(0, 0), part, lane);
  if constexpr (R == 2) load_groups<R, 8>(cb_k, 1, 0, lds + key_row_off<R>(1, 0), part, lane);
  {
    constexpr int kChunks = kPhaseBytes / 16;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.rope + kRopeFine32gOffset);
#pragma unroll
    for (int i = 0; i < kChunks / kThreads16; ++i) {
      const int c = (part * (kChunks / kThreads16) + i) * 64;
      __builtin_amdgcn_global_load_lds(src + (c + lane) * 16, lds + kPhaseOff + c * 16, 16, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const int nvalid = min(S, L - t0);
  const int nblocks = (nvalid + 63) >> 6;
  const int my_blocks = (nblocks - wave + kW - 1) / kW;  // this wave owns blocks wave, wave + kW, ...
  const int64_t row_base = seq_start + t0;
  // token row of block i for this lane, clamped into the split so every load is in bounds
  auto token_row = [&](int i) -> int64_t {
    int tl = (wave + kW * i) * 64 + lane;
    asm volatile("" : "+v"(tl));  // recomputed at every use rather than kept live
    return row_base + min(tl, nvalid - 1);
  };

  // (2) The query pairs this lane supplies to the broadcast A operand: head qi = lane mod 4, pairs
  // j = 16 k + quad (k = 0..3), and the coarse phases of those pairs for the wave's first block (row
  // t0 / 64 + wave) and for row 1 (e^{i 64 theta}, from which the per-block steps follow).
  const int quad = lane >> 2, qi = lane & 3;
  const f16* qp = static_cast<const f16*>(a.q) + (bh0 + qi) * kHeadDim;
  uint32_t qraw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) qraw[k] = *reinterpret_cast<const uint32_t*>(qp + 2 * (16 * k + quad));
  const float2* coarse = a.rope + kRopeCoarseOffset;
  const int last_row = (L - 1) >> 6;  // rows past the sequence are never read (the table may end there)
  const float2* crow0 = coarse + static_cast<int64_t>(min((t0 >> 6) + wave, last_row)) * kPairs;
  const float2* crow1 = coarse + static_cast<int64_t>(min(1, last_row)) * kPairs;
  float2 cph0[4], cph1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    cph0[k] = crow0[16 * k + quad];
    cph1[k] = crow1[16 * k + quad];
  }
  __builtin_amdgcn_sched_barrier(0);

  // (3) Key records of the first sweep (blocks 0, 1); later blocks' records are requested once the key pass has
  // started, so that they do not share the HBM queue with the first ones. Records are clamped rows, so every load
  // is in bounds.
  uint4 code[kMaxBlocks], code1[kMaxBlocks];  // residual 0 and (R = 2) residual 1 of each block
  auto request = [&](const uint8_t* base, int i) {
    code[i] = load_code_record(base, a.total_tokens, kv, token_row(i), R, 0);
    if constexpr (R == 2) code1[i] = load_code_record(base, a.total_tokens, kv, token_row(i), R, 1);
  };
#pragma unroll
  for (int i = 0; i < kSweep; ++i) request(a.k_codes, i);
  __builtin_amdgcn_sched_barrier(0);
  // (4) Key rows of groups 8-15 (and the R = 1 value codebook): published by the barrier before any wave reads
  // group 8 (publish_hi below).
  load_groups<R, 8>(cb_k, 0, 8, lds + key_row_off<R>(0, 8), part, lane);
  if constexpr (R == 2) {
    load_groups<R, 8>(cb_k, 1, 8, lds + key_row_off<R>(1, 8), part, lane);
  } else {
    load_groups<R, 16>(cb_v, 0, 0, lds + value_row_off<R>(0, 0), part, lane);
  }
  constexpr int kHiLoads = kStagedTables<R> ? (R == 2 ? 2 * 8 : 8 + 16) * kCodes / kThreads16 : 0;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kHiLoads));
  slot_barrier();  // every wave's groups 0-7, phases, query, coarse rows and first records have landed
  // Publishes the loads issued in (4): each wave waits for its own (n = loads it has issued since), then the
  // barrier. Called once by every wave, before its first read of group 8.
  auto publish_hi = [&](auto nc) {
    if constexpr (kStagedTables<R>) {
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most(decltype(nc)::value));
      slot_barrier();
    }
  };
  // R = 2: once every wave is past group 7 of its last key unit, region A is refilled with the value rows of
  // groups 0-7. Called once by every wave.
  auto refill_lo = [&]() {
    if constexpr (R == 2) {
      slot_barrier();
      load_groups<R, 8>(cb_v, 0, 0, lds + value_row_off<R>(0, 0), part, lane);
      load_groups<R, 8>(cb_v, 1, 0, lds + value_row_off<R>(1, 0), part, lane);
    }
  };

  // A operands. q'' = q * conj(e^{i 64 c theta}) for the block's coarse row c, in fp32: qc0 for the wave's
  // first block; stepE = e^{i 512 theta} (row 1 squared three times: the wave's blocks are 8 rows apart)
  // takes q'' from one block to the next.
  float2 qc0[4], stepE[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    asm volatile("" : "+v"(qraw[k]));
    const h2 hq = as_h2(qraw[k]);
    qc0[k] = cmul_conj(make_float2(static_cast<float>(hq.x), static_cast<float>(hq.y)), cph0[k]);
    float2 e = cph1[k];
#pragma unroll
    for (int sq = 0; sq < 3; ++sq) e = make_float2(e.x * e.x - e.y * e.y, 2.f * e.x * e.y);
    stepE[k] = e;
  }
  // base registers: kHiBase, and this lane's phase column (the fp32 phases of pairs 4g + 2h, 4g + 2h + 1 at
  // lane f sit at kPhaseOff + ((2g + h) * 64 + f) * 16)
  int hi = kHiBase, ph_lane = kPhaseOff + lane * 16;
  asm volatile("" : "+v"(hi), "+v"(ph_lane));

  // ------------------------------------------------------------------------------ key pass
  const h4 ident = identity_b(lane);  // identity MFMA operand (residual sums, transposes)
  f4 sc[kMaxBlocks];
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) sc[i] = (f4){0.f, 0.f, 0.f, 0.f};
  auto load_phases = [&](auto gc, float4 (&dst)[2]) {
    constexpr int g = decltype(gc)::value;
    dst[0] = *reinterpret_cast<const float4*>(lds + ph_lane + (2 * g) * 1024);
    dst[1] = *reinterpret_cast<const float4*>(lds + ph_lane + (2 * g + 1) * 1024);
  };
  auto key_rows = [&](auto gc, const uint4& c0, const uint4& c1, uint4 (&dst)[2]) {
    constexpr int g = decltype(gc)::value;
    dst[0] = lds_row<key_row_off<R>(0, g)>(lds, hi, code_index(c0, g));
    if constexpr (R == 2) dst[1] = lds_row<key_row_off<R>(1, g)>(lds, hi, code_index(c1, g));
  };
  // One sweep: groups 0..15 over blocks kSweep s, kSweep s + 1. Per group the two rotations run as one VALU burst,
  // then the next group's gathers and phases go out (the rows are consumed), then the 16 MFMAs as one burst over two
  // accumulators, covering the gathers' latency. The wave's issue priority falls as it progresses, so the two waves
  // that share a SIMD advance together.
  auto sweep = [&](auto sc_) {
    constexpr int s = decltype(sc_)::value;
    uint4 rows[kSweep][2];
    float4 ph[2];
    float2 A[kSweep];
    auto issue = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g < kGroups) {
        load_phases(gc, ph);
#pragma unroll
        for (int ii = 0; ii < kSweep; ++ii) key_rows(gc, code[kSweep * s + ii], code1[kSweep * s + ii], rows[ii]);
      }
    };
    // before group 8's rows: sweep 0 publishes the high rows; the last sweep hands region A to the value rows
    auto at_group8 = [&]() {
      if constexpr (s == 0) publish_hi(std::integral_constant<int, kSweep * R>{});
      if constexpr (s == kMaxBlocks / kSweep - 1) refill_lo();
    };
    f4 acc[2 * kSweep];  // two chains per block, folded into sc at the end of the sweep
#pragma unroll
    for (int c = 0; c < 2 * kSweep; ++c) acc[c] = (f4){0.f, 0.f, 0.f, 0.f};
    issue(std::integral_constant<int, 0>{});
    static_for<kGroups>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g % 4 == 0) {
        __builtin_amdgcn_s_setprio(3 - (kGroups * s + g) * 4 / (kGroups * (kMaxBlocks / kSweep)));
        // A operands of pairs 16 (g / 4) + quad for the sweep's blocks: q'' of block i is the first block's q''
        // stepped i times. qc0[k] holds q'' of the sweep's first block and is stepped on past the sweep's blocks
        // here (the same products in the same order as stepping from block 0 each time)
        constexpr int k = g / 4;
        float2 cur = qc0[k];
#pragma unroll
        for (int j = 0; j < kSweep; ++j) {
          A[j] = cur;
          cur = cmul_conj(cur, stepE[k]);
        }
        qc0[k] = cur;
      }
      float w[kSweep][8];
      if constexpr (R == 1) {
#pragma unroll
        for (int ii = 0; ii < kSweep; ++ii) rotate_f16(rows[ii][0], ph[0], ph[1], w[ii]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (g == 7) at_group8();
        issue(std::integral_constant<int, g + 1>{});  // the rows are consumed
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // the blocks' residual sums on the matrix core read the rows; the next group's gathers then go out ahead
        // of the rotations
        f4 ksum[kSweep][2];
        const float4 p0 = ph[0], p1 = ph[1];
#pragma unroll
        for (int ii = 0; ii < kSweep; ++ii) sum_rows(rows[ii][0], rows[ii][1], ident, ksum[ii]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (g == 7) at_group8();
        issue(std::integral_constant<int, g + 1>{});
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ii = 0; ii < kSweep; ++ii) rotate_f32(ksum[ii], p0, p1, w[ii]);
      }
      __builtin_amdgcn_sched_barrier(0);
      contract_key<g, kSweep>(w, A, acc);
      __builtin_amdgcn_sched_barrier(0);  // the fp32 MFMAs stay one burst, apart from the next VALU burst
    });
#pragma unroll
    for (int ii = 0; ii < kSweep; ++ii) sc[kSweep * s + ii] = acc[2 * ii] + acc[2 * ii + 1];
  };
  // One block alone (waves with an odd number of blocks): groups 0..15 with the phases read per group.
  float2 curA[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) curA[k] = qc0[k];
  auto single = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if (i < my_blocks) {
      uint4 rows[2];
      float4 ph[2];
      auto issue = [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        if constexpr (g < kGroups) {
          load_phases(gc, ph);
          key_rows(gc, code[i], code1[i], rows);
        }
      };
      issue(std::integral_constant<int, 0>{});
      f4 acc[2] = {(f4){0.f, 0.f, 0.f, 0.f}, (f4){0.f, 0.f, 0.f, 0.f}};  // real and imaginary chains
      static_for<kGroups>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        float w[1][8];
        rotate_key<R>(rows[0], rows[1], ph[0], ph[1], ident, w[0]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (g == 7) {
          if constexpr (i == 0) publish_hi(std::integral_constant<int, (kMaxBlocks - kSweep) * R>{});
          if (i == my_blocks - 1) refill_lo();
        }
        issue(std::integral_constant<int, g + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        const float2 A1[1] = {curA[g / 4]};
        contract_key<g, 1>(w, A1, acc);
        __builtin_amdgcn_sched_barrier(0);
      });
      sc[i] = acc[0] + acc[1];  // (a single block: the two chains)
#pragma unroll
      for (int k = 0; k < 4; ++k) curA[k] = cmul_conj(curA[k], stepE[k]);
    }
    // the block's key records are consumed: the value records of the first four blocks follow (the others are
    // requested during the value pass, four blocks ahead)
    if constexpr (i < kValueLead) request(a.v_codes, i);
  };
  if (my_blocks > 0 && my_blocks % kSweep == 0) {
    // each sweep first requests the next sweep's key records; the value records of the first four blocks follow
    // their key records. A wave with fewer than 8 blocks skips the sweeps past its blocks but issues the same
    // record loads (clamped rows), so that every vmcnt count below holds, and takes part in the region A
    // hand-over where its last sweep would have.
    static_for<kMaxBlocks / kSweep>([&](auto sc_) {
      constexpr int s = decltype(sc_)::value;
      if constexpr (kSweep * (s + 1) < kMaxBlocks) {
#pragma unroll
        for (int i = kSweep * (s + 1); i < kSweep * (s + 2); ++i) request(a.k_codes, i);
      }
      if (kSweep * s < my_blocks) {
        sweep(sc_);
      } else if constexpr (s == kMaxBlocks / kSweep - 1) {
        refill_lo();
      }
      if constexpr (kSweep * (s + 1) <= kValueLead) {
#pragma unroll
        for (int i = kSweep * s; i < kSweep * (s + 1); ++i) request(a.v_codes, i);
      }
    });
  } else {
#pragma unroll
    for (int i = kSweep; i < kMaxBlocks; ++i) request(a.k_codes, i);
    if (my_blocks == 0) {  // a wave without tokens still takes part in both hand-overs
      publish_hi(std::integral_constant<int, (kMaxBlocks - kSweep) * R>{});
      refill_lo();
    }
    static_for<kMaxBlocks>(single);
  }
  __builtin_amdgcn_s_setprio(0);

  // R = 2: once every wave is done with the key rows of groups 8-15 (and its region A value loads have landed),
  // region B is refilled with the value rows of groups 8-15; they are published inside the value pass.
  if constexpr (R == 2) {
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    slot_barrier();
    load_groups<R, 8>(cb_v, 0, 8, lds + value_row_off<R>(0, 8), part, lane);
    load_groups<R, 8>(cb_v, 1, 8, lds + value_row_off<R>(1, 8), part, lane);
  }

  // ------------------------------------------------------------------------------ wave softmax
  float m_w[kGqa], l_w[kGqa];
  wave_softmax_regs<kW>(sc, my_blocks, wave, lane, nvalid, a.scale, m_w, l_w);
  // p^T operands: lane 4b + j holds head j's weights for the 4 tokens of its quad (an exact transpose of the
  // fp16 weights through an identity MFMA)
  h4 pt[kMaxBlocks];
  {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) pt[i] = to_h4(mfma(to_h4(sc[i]), ident, z));
  }

  // ------------------------------------------------------------------------------ value pass
  f4 O[2 * kGroups];
#pragma unroll
  for (int c = 0; c < 2 * kGroups; ++c) O[c] = (f4){0.f, 0.f, 0.f, 0.f};
  if constexpr (R == 2) {
    // Units are (block, group pair); pairs 0-3 read region A, pairs 4-7 region B. Order: blocks 0 and 1 on pairs
    // 0-3, then (region B published) blocks 0 and 1 on pairs 4-7, then blocks 2..7 whole. Per unit the four rows of
    // both residuals go out kAhead units ahead of the arithmetic.
    constexpr int kPairsPerBlock = kGroups / 2;
    constexpr int kUnits = kPairsPerBlock * kMaxBlocks;
    constexpr int kLoUnits = 2 * kPairsPerBlock / 2;  // units before the region B hand-over
    auto unit_block = [](int u) {
      return u < 2 * kPairsPerBlock ? (u % kPairsPerBlock) / (kPairsPerBlock / 2) : u / kPairsPerBlock;
    };
    auto unit_pair = [](int u) {
      return u < 2 * kPairsPerBlock ? (u / kPairsPerBlock) * (kPairsPerBlock / 2) + u % (kPairsPerBlock / 2)
                                    : u % kPairsPerBlock;
    };
    uint4 rows[kBufs][2][2];  // [buffer][group of the pair][residual]
    auto issue = [&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < kUnits) {
        constexpr int i = unit_block(u), p = unit_pair(u);
        rows[u % kBufs][0][0] = lds_row<value_row_off<R>(0, 2 * p)>(lds, hi, code_index(code[i], 2 * p));
        rows[u % kBufs][0][1] = lds_row<value_row_off<R>(1, 2 * p)>(lds, hi, code_index(code1[i], 2 * p));
        rows[u % kBufs][1][0] = lds_row<value_row_off<R>(0, 2 * p + 1)>(lds, hi, code_index(code[i], 2 * p + 1));
        rows[u % kBufs][1][1] = lds_row<value_row_off<R>(1, 2 * p + 1)>(lds, hi, code_index(code1[i], 2 * p + 1));
      }
    };
    if (my_blocks > 0) static_for<kAhead>(issue);
    static_for<kUnits>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int i = unit_block(u), p = unit_pair(u);
      // a block's value records: block i asks for those of block i + kValueLead when it starts
      constexpr bool kFirstOfBlock = u < 2 * kPairsPerBlock ? u % kPairsPerBlock == 0 || u == kPairsPerBlock / 2
                                                            : u % kPairsPerBlock == 0;
      if constexpr (kFirstOfBlock && i + kValueLead < kMaxBlocks) request(a.v_codes, i + kValueLead);
      if constexpr (u == kLoUnits) {
        // region B: each wave's value loads (issued before the records of blocks 4 and 5), then the barrier
        publish_hi(std::integral_constant<int, 2 * R>{});
        if (my_blocks > 0) static_for<kAhead>([&](auto jc) { issue(std::integral_constant<int, u + decltype(jc)::value>{}); });
      }
      if (i < my_blocks) {
        __builtin_amdgcn_s_setprio(block_prio(u / kPairsPerBlock));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (u + kAhead < kLoUnits || u >= kLoUnits) issue(std::integral_constant<int, u + kAhead>{});
        __builtin_amdgcn_sched_barrier(0);
        value_pair2<p>(rows[u % kBufs], ident, pt[i], O);
      }
    });
  } else {
    const unsigned char* vtab = lds + hi;
    uint4 rows[kBufs][4];  // gathered rows of quarters n .. n + kAhead (4 groups each)
    auto issue = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 4 * kMaxBlocks) {
        constexpr int Q = m % 4;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          rows[m % kBufs][u] = *reinterpret_cast<const uint4*>(vtab + (4 * Q + u) * kCodes * 16 +
                                                               code_index(code[m / 4], 4 * Q + u) * 16);
      }
    };
    if (my_blocks > 0) static_for<kAhead>(issue);
    static_for<kMaxBlocks>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_s_setprio(block_prio(i));
      if constexpr (i + kValueLead < kMaxBlocks) request(a.v_codes, i + kValueLead);
      if (i < my_blocks) {
        static_for<4>([&](auto qc) {
          constexpr int n = 4 * i + decltype(qc)::value;
          __builtin_amdgcn_sched_barrier(0);
          issue(std::integral_constant<int, n + kAhead>{});
          __builtin_amdgcn_sched_barrier(0);
          static_for<4>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            value_step_quad<4 * (n % 4) + u>(rows[n % kBufs][u], ident, pt[i], O);
          });
        });
      }
    });
  }
  __builtin_amdgcn_s_setprio(0);

  // ------------------------------------------------------------------------ workgroup reduction
  attn_epilogue<kW>(a, lds, wave_ml, is_last, lane_id(), wave * 64 + lane_id(), wave, O, b, kv, split, L, S, bh0,
                    out_bh, m_w, l_w);
}

}  // namespace

hipError_t launch_attn_f16(int R, int B, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_splits * a.n_kv_heads, B);
  if (R == 1) attn_f16_kernel<1><<<grid, kThreads16, 0, s>>>(a);
  else attn_f16_kernel<2><<<grid, kThreads16, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace commvq
