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
// Work item: one workgroup per (sequence b, KV head, split of `split_tokens` tokens), one workgroup per
// CU (it owns the CU's LDS). Each wave owns 64-token blocks; lane = token within the block, so the fine
// RoPE phase e^{i (t mod 64) theta_j} is a per-lane constant held in registers (64 packed fp16 pairs).
//
// Phases K residual 0..R-1, then V residual 0..R-1, each a pass over the split's blocks with that
// residual's codebook (16 groups x 256 codes x 8 values) in LDS. fp16 storage keeps two 64 KiB codebook
// slots: while a phase runs on one slot, the next phase's codebook streams into the other by direct
// global->LDS loads, and the next phase's 16-byte code records stream into registers, so a phase
// boundary is one workgroup barrier. fp32 storage uses one 128 KiB slot and loads between phases.
//   K phase: gather the token's 16 codewords (one ds_read_b128 each), rotate them by the fine phase
//            (2 packed-fp16 ops per pair), and form the 4 GQA head scores with v_mfma_f32_4x4x4_16b_f16:
//            B = the token's rotated key (4 dims per step), A = the query rotated by the conjugate coarse
//            phase of the block, broadcast from one 4-lane block (CBSZ/ABID) so each lane supplies only
//            4 of the 64 query pairs. Scores accumulate across residuals in the MFMA accumulator.
//   softmax: per wave, m_w = max and l_w = sum of p = e^{s - m_w} over the wave's tokens; no barrier.
//   V phase: gather value codewords, transpose each 4x4 (token x dim) tile of a lane quad with an
//            identity-B MFMA, and accumulate p^T x v with the same 4x4x4 MFMA (the reduction over tokens
//            runs inside each quad; the 16 quads are summed once at the end).
// The workgroup then combines its waves (rescaling wave w by e^{m_w - M}), writes (M, L, o[128]) per q
// head, and the last workgroup of each (b, kv) (arrival counter in the workspace, reset to zero by that
// workgroup) merges the splits and writes out.
//
// fp32 storage uses the same structure with each fp32 operand split into fp16 hi + lo parts (three MFMA
// products per step) and the fine phase read from the fp32 table.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>
#include <utility>

#include "attn_common.h"

namespace commvq {
namespace {

// Per storage type: waves per workgroup and codebook slots in LDS.
template <typename T>
struct Shape;
template <>
struct Shape<f16> {
  static constexpr int kWaves = 8, kSlots = 2;
};
template <>
struct Shape<float> {
  static constexpr int kWaves = 4, kSlots = 1;
};

// ------------------------------------------------------------------ fp32 storage: per-group steps
// Key step for group G of one 64-token block: gather, rotate, MFMA steps (4 dims each). The fp16 path
// below processes groups in explicitly pipelined units instead.
template <int G, typename T>
struct KeyGroup;

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

// ------------------------------------------------------- fp16: explicitly pipelined block processing
// A block's 16 groups are processed in units (quarters of 4 groups, or pairs of groups with both residual
// rows); the gathers of a later unit are issued in a scheduling region ahead of the current unit's
// arithmetic (see kAhead), so each wave keeps LDS reads in flight while it rotates and multiplies.
template <int G>
__device__ __forceinline__ uint4 gather_row(const unsigned char* tab, const uint4& code) {
  return *reinterpret_cast<const uint4*>(tab + G * kCodes * 16 + code_index(code, G) * 16);
}
template <int Q>
__device__ __forceinline__ void gather_quarter(const unsigned char* tab, const uint4& code, uint4 (&buf)[4]) {
  buf[0] = gather_row<4 * Q + 0>(tab, code);
  buf[1] = gather_row<4 * Q + 1>(tab, code);
  buf[2] = gather_row<4 * Q + 2>(tab, code);
  buf[3] = gather_row<4 * Q + 3>(tab, code);
}
template <int Q>
__device__ __forceinline__ void key_quarter(const uint4 (&buf)[4], const uint4 (&F)[kGroups], const h4& A0,
                                            const h4& A1, f4& acc_even, f4& acc_odd) {
  key_step<4 * Q + 0>(buf[0], F, A0, A1, acc_even);  // two independent MFMA accumulation chains
  key_step<4 * Q + 1>(buf[1], F, A0, A1, acc_odd);
  key_step<4 * Q + 2>(buf[2], F, A0, A1, acc_even);
  key_step<4 * Q + 3>(buf[3], F, A0, A1, acc_odd);
}
// Fused residual key path (fp16, R = 2, both key codebooks resident): a block's groups go in pairs. Each
// group's two residual rows are gathered and summed in fp16; the rotation is linear, so the sum is rotated
// and multiplied once instead of once per residual.
template <int P>
__device__ __forceinline__ void gather_pair2(const unsigned char* tab0, const unsigned char* tab1, const uint4& c0,
                                             const uint4& c1, uint4 (&buf)[2][2]) {
  buf[0][0] = gather_row<2 * P>(tab0, c0);
  buf[0][1] = gather_row<2 * P>(tab1, c1);
  buf[1][0] = gather_row<2 * P + 1>(tab0, c0);
  buf[1][1] = gather_row<2 * P + 1>(tab1, c1);
}
template <int P>
__device__ __forceinline__ void key_pair2(const uint4 (&buf)[2][2], const uint4 (&F)[kGroups], const h4& A0,
                                          const h4& A1, f4& acc_even, f4& acc_odd) {
  key_step<2 * P>(add_rows(buf[0][0], buf[0][1]), F, A0, A1, acc_even);
  key_step<2 * P + 1>(add_rows(buf[1][0], buf[1][1]), F, A0, A1, acc_odd);
}
// Value path: each group's codeword row (8 dims) is gathered as two transposing 8-byte reads, which
// deliver the B operands of p^T x v directly: lane 4b + e gets dim e (and 4 + e) of the 4 tokens of
// MFMA block b (the tokens of lanes 16g + 4k + a). The p^T operand uses the same token grouping.
template <int Q>
__device__ __forceinline__ void gather_quarter_tr(const unsigned char* tab, const uint4& code, uint4 (&buf)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const unsigned char* row = tab + (4 * Q + u) * kCodes * 16 + code_index(code, 4 * Q + u) * 16;
    const h4 lo = lds_read_tr(row), hi = lds_read_tr(row + 8);
    buf[u] = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                        __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
  }
}
template <int G>
__device__ __forceinline__ void value_step(const uint4& tv, const h4& pt, f4 (&O)[2 * kGroups]) {
  O[2 * G] = mfma(pt, cat(as_h2(tv.x), as_h2(tv.y)), O[2 * G]);
  O[2 * G + 1] = mfma(pt, cat(as_h2(tv.z), as_h2(tv.w)), O[2 * G + 1]);
}
template <int Q>
__device__ __forceinline__ void value_quarter(const uint4 (&buf)[4], const h4& pt, f4 (&O)[2 * kGroups]) {
  value_step<4 * Q + 0>(buf[0], pt, O);
  value_step<4 * Q + 1>(buf[1], pt, O);
  value_step<4 * Q + 2>(buf[2], pt, O);
  value_step<4 * Q + 3>(buf[3], pt, O);
}

// Fused residual value path (fp16, R = 2, both value codebooks resident): each group's two residual rows
// are gathered whole (16 bytes each: a random 16-byte LDS gather costs less than two transposing 8-byte
// reads) and summed in fp16. An MFMA against the identity then transposes each 4-dim half within its quad
// of lanes: lane 4b + j receives dim j of the quad's 4 tokens (exactly, in fp32), which converted back is
// the B operand of p^T x v for MFMA block b = the quad. The p^T operand uses the same quad grouping.
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

// fp32 storage: a block's 16 groups in sequence.
template <typename T, int Base, typename... Args, int... Gs>
__device__ __forceinline__ void key_seq(std::integer_sequence<int, Gs...>, Args&&... args) {
  (KeyGroup<Base + Gs, T>::run(args...), ...);
}
template <typename T, int Base, typename... Args, int... Gs>
__device__ __forceinline__ void value_seq(std::integer_sequence<int, Gs...>, Args&&... args) {
  (ValueGroup<Base + Gs, T>::run(args...), ...);
}
template <typename T, typename... Args>
__device__ __forceinline__ void key_groups(Args&&... args) {
  key_seq<T, 0>(std::make_integer_sequence<int, kGroups>{}, args...);
}
template <typename T, typename... Args>
__device__ __forceinline__ void value_groups(Args&&... args) {
  value_seq<T, 0>(std::make_integer_sequence<int, kGroups>{}, args...);
}

template <typename T, int R>
__global__ void __launch_bounds__(Shape<T>::kWaves * 64) attn_kernel(const AttnArgs a) {
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr int kW = Shape<T>::kWaves;
  constexpr int kThreads = kW * 64;
  constexpr int kSlots = Shape<T>::kSlots;
  constexpr int kTab = kGroups * kCodes * kGroupDim * static_cast<int>(sizeof(T));
  constexpr int kPhases = 2 * R;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kSlots * kTab];
  __shared__ __attribute__((aligned(16))) uint4 fine_lds[kF32 ? 1 : kGroups * kFineRows];  // fp16 fine phases
  __shared__ float wave_ml[2][kW][kGqa];  // per wave and head: softmax max m_w and sum l_w
  __shared__ __attribute__((aligned(16))) uint2 p_scratch[kF32 ? 1 : kW][64];  // fp16: p^T transposes
  __shared__ int is_last;

  // XCD-aware work order: the KV head is the fastest grid index. Workgroups are dealt to the 8 XCDs in
  // turn, so with 8 KV heads each XCD serves one head and its L2 fetches only that head's codebooks.
  const int kv = blockIdx.x % a.n_kv_heads, split = blockIdx.x / a.n_kv_heads, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave values scalar
  const int64_t cb_stride = static_cast<int64_t>(kGroups) * R * kCodes * kGroupDim;
  const T* cb_k = static_cast<const T*>(a.k_cb) + kv * cb_stride;
  const T* cb_v = static_cast<const T*>(a.v_cb) + kv * cb_stride;
  auto table_src = [&](int p) { return p < R ? cb_k : cb_v; };
  // sequence bounds (clamped), read before any memory operation so that they stay scalar loads
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.max_len, a.total_tokens);
  const int L = sb.len;
  const int64_t seq_start = sb.start;

  // ---------------------------------------------------------------------------------- prologue
  // (1) The codebooks of the first phases and (fp16 storage) the group-major packed-fp16 fine phases
  // (16 KiB, once per workgroup; every wave then reads its lane's 64 phases from LDS), straight into LDS.
  // They depend on nothing but the KV head, so they go out before the sequence bounds have arrived.
  if constexpr (!kF32) {
    constexpr int kFineChunks = kGroups * kFineRows;  // 16-byte entries
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.rope + kRopeFine16Offset);
#pragma unroll
    for (int i = 0; i < kFineChunks / kThreads; ++i) {
      const int c = (wave * (kFineChunks / kThreads) + i) * 64;
      __builtin_amdgcn_global_load_lds(src + (c + lane) * 16, reinterpret_cast<unsigned char*>(fine_lds) + c * 16, 16,
                                       0, 0);
    }
  }
#pragma unroll
  for (int p = 0; p < (kSlots < kPhases ? kSlots : kPhases); ++p)
    load_table<T, R, kW>(table_src(p), p % R, lds + p * kTab, wave, lane);
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

  // (2) register operands the first block needs: query pairs, coarse phases of every block, fine phases.
  // Query pairs this lane supplies to the broadcast A operand: head qi, pairs 2*quad + {0,1} (+32).
  const int quad = lane >> 2, qi = lane & 3;
  const T* qp = static_cast<const T*>(a.q) + (bh0 + qi) * kHeadDim;
  // raw query pairs (converted after the prologue barrier): index 2m + e is pair 32m + 2 quad + e
  typedef typename std::conditional<kF32, float2, uint32_t>::type QPair;
  QPair qraw[4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) qraw[2 * m + e] = *reinterpret_cast<const QPair*>(qp + 2 * (32 * m + 2 * quad + e));
  const float2* coarse = a.rope + kRopeCoarseOffset;
  // Coarse phases of this lane's 4 query pairs (index 2m + e: pair 32m + 2 quad + e). fp32 storage: one
  // row per block. fp16 storage: the row of the wave's first block and row 1 (e^{i 64 theta}), from
  // which the per-block rotation steps follow (below).
  constexpr int kCoarseRows = kF32 ? kMaxBlocks : 2;
  float4 cphase[kCoarseRows][2];
#pragma unroll
  for (int i = 0; i < kCoarseRows; ++i) {
    // clamped rows: never past the sequence, so always inside the table
    const int row = kF32 ? (t0 >> 6) + min(wave + kW * i, nblocks - 1) : (i == 0 ? (t0 >> 6) + wave : min(1, (L - 1) >> 6));
    const float2* cr = coarse + static_cast<int64_t>(kF32 || i == 1 ? row : min(row, (L - 1) >> 6)) * kPairs;
#pragma unroll
    for (int m = 0; m < 2; ++m) cphase[i][m] = *reinterpret_cast<const float4*>(cr + 32 * m + 2 * quad);
  }
  const float2* fine = a.rope + lane;  // fp32 storage: fine[j * 64 + lane], read per group
  __builtin_amdgcn_sched_barrier(0);
  // (3) code records of phase 0. Code records of the current phase live in code[]; once a block has
  // consumed its record, the record of the same token for the next phase is requested. Every phase
  // issues exactly kMaxBlocks record loads per wave (clamped rows), so a fixed vmcnt finds the codebook
  // loads issued before them.
  uint4 code[kMaxBlocks];
  auto request_codes = [&](int ph, int i) {
    const uint8_t* base = ph < R ? a.k_codes : a.v_codes;
    code[i] = load_code_record(base, a.total_tokens, kv, token_row(i), R, ph % R);
  };
  // fp16, R = 2: both key codebooks are resident from the start, so both residuals' key records of a
  // block are consumed together by one fused key pass (code[] holds residual 0, code1[] residual 1)
  constexpr bool kFusedKey = !kF32 && R == 2;
  uint4 code1[kMaxBlocks];
  // The prologue requests the records of the first kLeadBlocks blocks only (a wave's full share would
  // queue a large part of the whole code stream ahead of the codebook loads); block i of the first phase
  // requests block i + kLeadBlocks.
  constexpr int kLeadBlocks = kMaxBlocks < 3 ? kMaxBlocks : 3;
  auto request_key_records = [&](int i) {
    request_codes(0, i);
    if constexpr (kFusedKey) code1[i] = load_code_record(a.k_codes, a.total_tokens, kv, token_row(i), R, 1);
  };
#pragma unroll
  for (int i = 0; i < kLeadBlocks; ++i) request_key_records(i);
  constexpr int kPrologueRecords = (kFusedKey ? 2 : 1) * kLeadBlocks;

  // Codebooks of phases 2 and 3 (fp16, R = 2) cannot be loaded up front (both slots are busy), so during
  // phase p the codebook of phase p + 1 is staged through registers into the slot phase p - 1 used: one
  // 16-byte row per thread per block, written to LDS one block later. (A direct global->LDS load here
  // would make the compiler wait for it before every LDS read of the other slot.)
  auto slot_of = [&](int p) { return lds + (p % kSlots) * kTab; };
  auto staged = [](int p) { return kSlots == 2 && p >= 1 && p + 1 < kPhases; };
  uint4 stage;
  auto stage_load = [&](int pn, int i) {  // row i * kThreads + tid of phase pn's codebook
    const int row = i * kThreads + tid, g = row >> 8, l = row & (kCodes - 1);
    stage = *reinterpret_cast<const uint4*>(table_src(pn) + ((static_cast<int64_t>(g) * R + pn % R) * kCodes + l) *
                                                                kGroupDim);
  };
  auto stage_store = [&](int pn, int i) {
    *reinterpret_cast<uint4*>(slot_of(pn) + (i * kThreads + tid) * 16) = stage;
  };
  static_assert(kSlots == 1 || kTab / 16 == kMaxBlocks * kThreads, "one staged codebook row per thread per block");

  // End of phase p: make the codebook of phase p + 1 resident and visible.
  auto next_phase = [&](int p) {
    if constexpr (kSlots == 2) {
      if (staged(p)) stage_store(p + 1, kMaxBlocks - 1);
      // Codebook p+1 came with the prologue and slot p % 2 is never refilled (R = 1): each wave moves on
      // without waiting for the others.
      if (p + 1 < kSlots && p + 2 >= kPhases) return;
      lds_barrier();  // codebook p+1 complete (prologue load or staged rows); every wave is done with slot p % 2
    } else {
      slot_barrier();  // every wave is done with the slot
      load_table<T, R, kW>(table_src(p + 1), (p + 1) % R, lds, wave, lane);
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
      slot_barrier();
    }
  };
  // The first codebooks were issued before the code records, which the barrier keeps last. Nothing may
  // wait on a loaded register between the codebook loads and this point: while a direct-to-LDS load is
  // outstanding the compiler can only wait with vmcnt(0), which would include the records.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kPrologueRecords));
  slot_barrier();
  uint4 F[kGroups];  // fp16 storage: fine phases of pairs 4g..4g+3 at this lane's t mod 64 = lane
  if constexpr (!kF32) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) F[g] = fine_lds[g * kFineRows + lane];
  }
  // Pin the query and coarse-phase registers here, so the arithmetic on them (and its wait for their
  // loads) cannot be hoisted above the codebook loads.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (kF32) {
      asm volatile("" : "+v"(qraw[k].x), "+v"(qraw[k].y));
    } else {
      asm volatile("" : "+v"(qraw[k]));
    }
  }
#pragma unroll
  for (int i = 0; i < kCoarseRows; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
      asm volatile("" : "+v"(cphase[i][m].x), "+v"(cphase[i][m].y), "+v"(cphase[i][m].z), "+v"(cphase[i][m].w));
  float2 qv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (kF32) {
      qv[k] = qraw[k];
    } else {
      const h2 hq = as_h2(qraw[k]);
      qv[k] = make_float2(static_cast<float>(hq.x), static_cast<float>(hq.y));
    }
  }

  // A operands: the query rotated by the conjugate coarse phase of each 64-token block,
  // q'' = q * conj(C), in fp16 (fp32 inputs: hi and lo fp16 parts); the same for every key phase.
  // fp32 storage computes all of them here. fp16 storage keeps q''_0 of the wave's first block and the
  // step E = e^{i 64 kW theta} (row 1 squared log2(kW) times): the wave's blocks are kW rows apart, so
  // q''_{i+1} = q''_i * conj(E). Seven fp32 steps stay far below the fp16 rounding of the operand.
  h4 Ah[kF32 ? kMaxBlocks : 1][2], Al[kF32 ? kMaxBlocks : 1][2];
  float2 qc0[4], stepE[4];
  if constexpr (kF32) {
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
  } else {
    static_assert((kW & (kW - 1)) == 0, "blocks of a wave are a power-of-two number of rows apart");
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float4 c0 = cphase[0][m], c1 = cphase[1][m];
      qc0[2 * m] = cmul_conj(qv[2 * m], make_float2(c0.x, c0.y));
      qc0[2 * m + 1] = cmul_conj(qv[2 * m + 1], make_float2(c0.z, c0.w));
      stepE[2 * m] = make_float2(c1.x, c1.y);
      stepE[2 * m + 1] = make_float2(c1.z, c1.w);
    }
#pragma unroll
    for (int sq = 1; sq < kW; sq *= 2)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 e = stepE[k];
        stepE[k] = make_float2(e.x * e.x - e.y * e.y, 2.f * e.x * e.y);
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
    const unsigned char* tab = slot_of(r);
    float2 cur[4];  // fp16 storage: q'' of the current block
#pragma unroll
    for (int k = 0; k < 4; ++k) cur[k] = qc0[k];
    uint4 rows[kBufs][4];  // fp16: gathered rows of quarters n .. n + kAhead
    auto issue = [&](auto mc) {  // gathers of quarter m = 4 * block + q (clamped records: always in bounds)
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 4 * kMaxBlocks) gather_quarter<m % 4>(tab, code[m / 4], rows[m % kBufs]);
    };
    if constexpr (!kF32) {
      if (my_blocks > 0) static_for<kAhead>(issue);
    }
    auto key_block = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (!kF32) __builtin_amdgcn_s_setprio(block_prio(i));
      if constexpr (r == 0 && i + kLeadBlocks < kMaxBlocks) request_key_records(i + kLeadBlocks);
      if constexpr (staged(r)) {
        if (i > 0) stage_store(r + 1, i - 1);
        stage_load(r + 1, i);
      }
      if (i < my_blocks) {
        if constexpr (!kF32) {
          const h4 A0 = {(f16)cur[0].x, (f16)cur[0].y, (f16)cur[1].x, (f16)cur[1].y};
          const h4 A1 = {(f16)cur[2].x, (f16)cur[2].y, (f16)cur[3].x, (f16)cur[3].y};
          f4 odd = {0.f, 0.f, 0.f, 0.f};
          auto quarter = [&](auto qc) {
            constexpr int n = 4 * i + decltype(qc)::value;
            __builtin_amdgcn_sched_barrier(0);
            issue(std::integral_constant<int, n + kAhead>{});
            __builtin_amdgcn_sched_barrier(0);
            key_quarter<n % 4>(rows[n % kBufs], F, A0, A1, sc[i], odd);
          };
          static_for<4>(quarter);
          sc[i] += odd;
#pragma unroll
          for (int k = 0; k < 4; ++k) cur[k] = cmul_conj(cur[k], stepE[k]);
        } else {
          key_groups<float>(tab, code[i], fine, Ah[i], Al[i], sc[i]);
        }
      }
      request_codes(r + 1, i);  // phase r + 1 always exists (the value phases follow)
    };
    static_for<kMaxBlocks>(key_block);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (r + 1 < R) next_phase(r);
  };
  // Fused pass (fp16, R = 2): per group pair, the four rows of both residuals go out ahead of the previous
  // pair's arithmetic; the records of the first value phase follow each block.
  auto fused_key_pass = [&]() {
    const unsigned char* tab0 = slot_of(0);
    const unsigned char* tab1 = slot_of(1);
    float2 cur[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) cur[k] = qc0[k];
    uint4 rows[kBufs][2][2];  // [buffer][group of the pair][residual]
    auto issue = [&](auto mc) {  // gathers of pair m = 8 * block + pair (clamped records: always in bounds)
      constexpr int m = decltype(mc)::value;
      constexpr int kPairs = kGroups / 2;
      if constexpr (m < kPairs * kMaxBlocks)
        gather_pair2<m % kPairs>(tab0, tab1, code[m / kPairs], code1[m / kPairs], rows[m % kBufs]);
    };
    if (my_blocks > 0) static_for<kAhead>(issue);
    auto key_block = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_s_setprio(block_prio(i));
      if constexpr (i + kLeadBlocks < kMaxBlocks) request_key_records(i + kLeadBlocks);
      if (i < my_blocks) {
        const h4 A0 = {(f16)cur[0].x, (f16)cur[0].y, (f16)cur[1].x, (f16)cur[1].y};
        const h4 A1 = {(f16)cur[2].x, (f16)cur[2].y, (f16)cur[3].x, (f16)cur[3].y};
        f4 odd = {0.f, 0.f, 0.f, 0.f};
        auto pair_step = [&](auto pc) {
          constexpr int n = (kGroups / 2) * i + decltype(pc)::value;
          __builtin_amdgcn_sched_barrier(0);
          issue(std::integral_constant<int, n + kAhead>{});
          __builtin_amdgcn_sched_barrier(0);
          key_pair2<n % (kGroups / 2)>(rows[n % kBufs], F, A0, A1, sc[i], odd);
        };
        static_for<kGroups / 2>(pair_step);
        sc[i] += odd;
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = cmul_conj(cur[k], stepE[k]);
      }
    };
    static_for<kMaxBlocks>(key_block);
    __builtin_amdgcn_s_setprio(0);
  };
  if constexpr (kFusedKey) {
    fused_key_pass();
  } else {
    key_phase(std::integral_constant<int, 0>{});
    if constexpr (R > 1) key_phase(std::integral_constant<int, 1>{});
  }
  // Fused passes: both slots held key codebooks, so the value codebooks could not be staged during the key
  // pass. Each thread fetches its 8 rows of each now (and the value records of the first blocks); the rows
  // are written once every wave is done with the key slots.
  constexpr int kRowsPerThread = kTab / 16 / kThreads;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // (a plain vector type keeps the rows in VGPRs)
  u32x4 vrows[2][kRowsPerThread];
  auto request_value_records = [&](int i) {
    code[i] = load_code_record(a.v_codes, a.total_tokens, kv, token_row(i), R, 0);
    code1[i] = load_code_record(a.v_codes, a.total_tokens, kv, token_row(i), R, 1);
  };
  if constexpr (kFusedKey) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int k = 0; k < kRowsPerThread; ++k) {
        const int row = k * kThreads + tid, g = row >> 8, l = row & (kCodes - 1);
        vrows[rr][k] =
            *reinterpret_cast<const u32x4*>(cb_v + ((static_cast<int64_t>(g) * R + rr) * kCodes + l) * kGroupDim);
      }
#pragma unroll
    for (int i = 0; i < kLeadBlocks; ++i) request_value_records(i);
  }

  // ------------------------------------------------------------------------------ wave softmax
  wave_softmax<kW>(sc, my_blocks, wave, lane, nvalid, a.scale, wave_ml);

  // p^T operands: lane 4b+j holds head j's weights for the 4 tokens of its quad (quad transpose)
  const h4 ident = identity_b(lane);
  h4 pth[kMaxBlocks], ptl[kMaxBlocks];
  {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      if constexpr (kFusedKey) {
        pth[i] = to_h4(mfma(to_h4(sc[i]), ident, z));  // quad grouping: an exact transpose of fp16 values
        ptl[i] = pth[i];
      } else if constexpr (!kF32) {
        // lane writes its token's 4 head weights (fp16); the transposing read returns, in lane 4b + e,
        // head e's weights of the 4 tokens of MFMA block b, matching the value operands
        p_scratch[wave][lane] = __builtin_bit_cast(uint2, to_h4(sc[i]));
        pth[i] = lds_read_tr(&p_scratch[wave][lane]);
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
  if constexpr (kFusedKey) {
    lds_barrier();  // every wave is done with both key codebooks
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int k = 0; k < kRowsPerThread; ++k)
        *reinterpret_cast<u32x4*>(slot_of(R + rr) + (k * kThreads + tid) * 16) = vrows[rr][k];
    lds_barrier();  // both value codebooks complete
  } else {
    next_phase(R - 1);
  }

  // ------------------------------------------------------------------------------ value phases
  f4 O[2 * kGroups];
#pragma unroll
  for (int c = 0; c < 2 * kGroups; ++c) O[c] = (f4){0.f, 0.f, 0.f, 0.f};
  auto value_phase = [&](auto rc) {
    constexpr int r = decltype(rc)::value;
    constexpr int p = R + r;
    const unsigned char* tab = slot_of(p);
    uint4 rows[kBufs][4];  // fp16: gathered rows of quarters n .. n + kAhead
    auto issue = [&](auto mc) {  // gathers of quarter m = 4 * block + q (clamped records: always in bounds)
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 4 * kMaxBlocks) gather_quarter_tr<m % 4>(tab, code[m / 4], rows[m % kBufs]);
    };
    if constexpr (!kF32) {
      if (my_blocks > 0) static_for<kAhead>(issue);
    }
    auto value_block = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (!kF32) __builtin_amdgcn_s_setprio(block_prio(i));
      if constexpr (staged(p)) {
        if (i > 0) stage_store(p + 1, i - 1);
        stage_load(p + 1, i);
      }
      if (i < my_blocks) {
        if constexpr (!kF32) {
          auto quarter = [&](auto qc) {
            constexpr int n = 4 * i + decltype(qc)::value;
            __builtin_amdgcn_sched_barrier(0);
            issue(std::integral_constant<int, n + kAhead>{});
            __builtin_amdgcn_sched_barrier(0);
            value_quarter<n % 4>(rows[n % kBufs], pth[i], O);
          };
          static_for<4>(quarter);
        } else {
          value_groups<T>(tab, code[i], ident, pth[i], ptl[i], O);
        }
      }
      if constexpr (r + 1 < R) request_codes(p + 1, i);
    };
    static_for<kMaxBlocks>(value_block);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (r + 1 < R) next_phase(p);
  };
  // Fused value pass (fp16, R = 2): per group pair, the four rows of both residuals go out ahead of the
  // previous pair's arithmetic; block i requests the records of block i + kLeadBlocks.
  auto fused_value_pass = [&]() {
    const unsigned char* tab0 = slot_of(R);
    const unsigned char* tab1 = slot_of(R + 1);
    uint4 rows[kBufs][2][2];  // [buffer][group of the pair][residual]
    auto issue = [&](auto mc) {  // gathers of pair m = 8 * block + pair (clamped records: always in bounds)
      constexpr int m = decltype(mc)::value;
      constexpr int kPairs = kGroups / 2;
      if constexpr (m < kPairs * kMaxBlocks)
        gather_pair2<m % kPairs>(tab0, tab1, code[m / kPairs], code1[m / kPairs], rows[m % kBufs]);
    };
    if (my_blocks > 0) static_for<kAhead>(issue);
    auto value_block = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_s_setprio(block_prio(i));
      if constexpr (i + kLeadBlocks < kMaxBlocks) request_value_records(i + kLeadBlocks);
      if (i < my_blocks) {
        auto pair_step = [&](auto pc) {
          constexpr int n = (kGroups / 2) * i + decltype(pc)::value;
          __builtin_amdgcn_sched_barrier(0);
          issue(std::integral_constant<int, n + kAhead>{});
          __builtin_amdgcn_sched_barrier(0);
          value_pair2<n % (kGroups / 2)>(rows[n % kBufs], ident, pth[i], O);
        };
        static_for<kGroups / 2>(pair_step);
      }
    };
    static_for<kMaxBlocks>(value_block);
    __builtin_amdgcn_s_setprio(0);
  };
  if constexpr (kFusedKey) {
    fused_value_pass();
  } else {
    value_phase(std::integral_constant<int, 0>{});
    if constexpr (R > 1) value_phase(std::integral_constant<int, 1>{});
  }

  // ------------------------------------------------------------------------ workgroup reduction
  // (Lane and thread indices are recomputed here so that no index register lives across the phases.)
  attn_epilogue<kW>(a, lds, wave_ml, is_last, lane_id(), wave * 64 + lane_id(), wave, O, b, kv, split, L, S, bh0,
                    out_bh);
}

}  // namespace

hipError_t launch_attn(int dtype, int R, int B, const AttnArgs& a, hipStream_t s) {
  if (dtype == COMMVQ_F16) return launch_attn_f16(R, B, a, s);
  dim3 grid(a.n_splits * a.n_kv_heads, B);
  constexpr int kThreads = Shape<float>::kWaves * 64;
  if (R == 1) attn_kernel<float, 1><<<grid, kThreads, 0, s>>>(a);
  else attn_kernel<float, 2><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace commvq
