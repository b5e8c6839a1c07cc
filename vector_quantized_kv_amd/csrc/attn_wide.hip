// Decode-step attention over a CommVQ cache in the pages' own code shape, on gfx950.
//
// Same computation as the byte-layout kernels
// (score = scale * sum_j Re(conj(q_j) khat_{t,j} e^{i t theta_j}),
// out = softmax-weighted sum of vhat), for the setting the CommVQ pages evaluate: one code index shared by
// the 64 dims of a half head (G = 2 groups of 64 dims), N = 64 codewords per residual codebook (6-bit
// indices), and many residual rounds. The average is R log2(N) / g bits per scalar (pith.science verdict
// for arXiv 2506.18879, key_machinery; its referee report's minor comments give g = 64, N' = 64), so
// R = 11 gives about 1 bit and R = 21 about 2 (the CommVQ summary page, Limitations, names these two).
// A token's R x G indices are one little-endian bitstream of 32-bit words, index (r, g) at bit 6 (r G + g);
// word w of every token of a KV head lies in word plane w ([Hkv][words][T]).
//
// The key codebooks (R x 16 KiB per KV head) do not fit in LDS, so the key side runs in passes. A pass holds
// 8 tables of 8 KiB (64 KiB) in one of two LDS slots while the next pass's tables are staged through registers
// into the other slot. Index window c of the bitstream (residuals kRes c .. kRes c + kRes - 1) takes two passes,
// one per group g, of kRes residuals each. The last window holds TAIL residuals (the kernel's template argument):
// one pass over both groups if TAIL <= kRes / 2, else two passes of TAIL residuals, so every pass gathers only
// rows of residuals that exist and no pass branches inside its units (a slot's unused tables hold zero rows).
// Scores are linear in the residuals, so each pass adds its share to the MFMA accumulators. The rotation and the
// contraction run once per pass and unit, so a pass over more residuals of one group costs less arithmetic per
// gathered row.
//
// Values take the pages' own form (pith.science verdict for arXiv 2506.18879, key_machinery and
// forward_implications: the softmax weights multiply the value codes before the codebook product): every
// token adds its softmax weights to bin (g, r, l) of each of its value indices, and the bins are contracted
// with the value codebook once per workgroup. A row gather moves 128 bytes per (token, residual, group); a
// bin update moves the 4 heads' weights in two 64-bit LDS atomics, about a third of the LDS time. The weights
// are e^{s - M} with M the workgroup's maximum per head, in fixed point (multiples of 2^-19, two heads per
// 64-bit bin whose 32-bit halves never carry into each other), so the bins are exact and independent of the
// order of the adds.
//
// Work item, lanes and MFMA layouts are those of the fp16 byte-layout kernel (attn_f16.hip): lane = token of a
// 64-token block, 4 GQA heads per KV head, the per-64-token RoPE phase on the query and the per-lane phase on
// the keys. A 16-byte chunk cc of the 128-byte row of group g holds RoPE pairs 32 g + 4 cc .. + 3, exactly
// the pairs of the byte layout's group 8 g + cc, so the key contraction's query operand and the epilogue are
// the byte layout's. Per unit (g, cc) a lane gathers its token's chunk from each of the pass's residual rows,
// sums them in fp32 on the matrix core (an MFMA with the identity as A adds a lane's four fp16 values to its
// fp32 accumulator), rotates the sum by the lane's fine phases in fp32 (phases read from a 32 KiB LDS table) and
// contracts it with the fp32 block query on the fp32 matrix core (v_mfma_f32_4x4x1_16b_f32, query broadcast
// from one 4-lane block per dim): no fp16 rounding on the key side, so wide logit ranges keep the attention
// within tolerance.
// Rows are stored with their 16-byte chunks permuted by the codeword (physical chunk = cc xor
// ((l >> 1) & 7)), so the 16 lanes that share an LDS cycle land on random ones of the 16 bank groups
// instead of the two that a 128-byte row stride would give them.
#include "attn_common.h"

namespace commvq {
namespace {

constexpr int kWG = kWideGroups;                 // index groups per head (2)
constexpr int kWN = kWideCodes;                  // codewords per residual codebook (64)
constexpr int kWRow = kHeadDim / kWG * 2;        // bytes per fp16 codeword row (128)
constexpr int kWTab = kWN * kWRow;               // bytes per (residual, group) table (8 KiB)
constexpr int kRes = kWideResPerPass;            // residuals per index window (8)
constexpr int kIdx = kRes * kWG;                 // indices per window (16)
constexpr int kTables = 8;                       // (residual, group) tables per codebook slot
constexpr int kSlot = kTables * kWTab;           // bytes per codebook slot (64 KiB)
constexpr int kChunks = kWRow / 16;              // 16-byte chunks per row (8)
constexpr int kW = 8;                            // waves per workgroup
constexpr int kThreads = kW * 64;
constexpr int kPhase = 2 * kSlot;                // LDS offset of the fp32 fine phases [G][h][lane][2 pairs]
constexpr int kPhaseBytes = kGroups * 2 * 64 * 16;
constexpr int kWAhead = 1;                       // units whose gathers are in flight ahead of the current one
constexpr int kWBufs = kWAhead + 1;
constexpr int kFxBits = 19;                      // value bins: softmax weights in multiples of 2^-19
static_assert(kSlot / 16 == kMaxBlocks * kThreads, "one staged 16-byte unit per thread per block");
static_assert(kPhase + kPhaseBytes <= 160 * 1024, "codebook slots and phases fit the CU's LDS");
static_assert(kWG * kWideMaxResiduals * 2 * kWN * 8 <= kSlot, "the value bins fit one codebook slot");
static_assert((static_cast<int64_t>(kW) * kMaxBlocks * 64 << kFxBits) <= (static_cast<int64_t>(1) << 32),
              "a bin's 32-bit halves (each at most 2^19 per token) never carry into each other");

// Global source of 16-byte unit u (0 .. 511) of the LDS table of residual r, group g: codeword l = u / 8, physical
// chunk pc = u % 8.
__device__ __forceinline__ const unsigned char* table_unit_src(const f16* cb_kv, int R, int g, int r, int u) {
  const int l = (u >> 3) & (kWN - 1), pc = u & 7;
  const int cc = pc ^ ((l >> 1) & 7);
  return reinterpret_cast<const unsigned char*>(cb_kv + ((static_cast<int64_t>(g) * R + r) * kWN + l) * (kWRow / 2)) +
         cc * 16;
}

// fp32 4x4x1 MFMA with the A operand broadcast from block ABID: acc[m] += A[lane 4 ABID + m] * b.
template <int ABID>
__device__ __forceinline__ f4 mfma32_bcast(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 4, ABID, 0);
}

// Key unit of byte-layout group G = 8 g + CC (RoPE pairs 4G .. 4G+3): the sum of the unit's NR residual chunks
// (zero rows past R), in fp32 on the matrix core (with A = identity, lane 4b + j of D receives its own B values
// plus C), rotated by the lane's fine phases (p0: pairs 4G, 4G+1; p1: 4G+2, 4G+3, each (cos, sin)) in fp32,
// then contracted with the block query q'' (pair j = 4G + u broadcast from block j mod 16, which does not
// depend on g): q''_re x w_re into acc[0], q''_im x w_im into acc[1].
template <int NR, int CC>
__device__ __forceinline__ void wide_key_unit(const uint4 (&rows)[NR], const h4& ident, const float4& p0,
                                              const float4& p1, const float2& A, f4 (&acc)[2]) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  f4 k0 = mfma(ident, cat(as_h2(rows[0].x), as_h2(rows[0].y)), z);
  f4 k1 = mfma(ident, cat(as_h2(rows[0].z), as_h2(rows[0].w)), z);
#pragma unroll
  for (int rho = 1; rho < NR; ++rho) {
    k0 = mfma(ident, cat(as_h2(rows[rho].x), as_h2(rows[rho].y)), k0);
    k1 = mfma(ident, cat(as_h2(rows[rho].z), as_h2(rows[rho].w)), k1);
  }
  const float cs[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  float w[8];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float c = cs[2 * u], s = cs[2 * u + 1];
    const float kr = (u < 2 ? k0 : k1)[2 * (u & 1)], ki = (u < 2 ? k0 : k1)[2 * (u & 1) + 1];
    w[2 * u] = fmaf(kr, c, -(ki * s));
    w[2 * u + 1] = fmaf(ki, c, kr * s);
  }
  __builtin_amdgcn_sched_barrier(0);  // the fp32 MFMAs run as one burst (they do not overlap VALU work)
  static_for<8>([&](auto dc) {
    constexpr int d = decltype(dc)::value;
    constexpr int abid = (4 * CC + d / 2) & 15;
    acc[d & 1] = mfma32_bcast<abid>((d & 1) ? A.y : A.x, w[d], acc[d & 1]);
  });
  __builtin_amdgcn_sched_barrier(0);
}

// One residual's share of the bins x value codebook product for RoPE-pair chunk CC of its group: the B operands
// (lane 4 q + j: dim 8 CC + 4 x + j of codewords 4 q .. 4 q + 3) come from the residual's table in LDS through
// the transposing read, where the table holds codeword l's chunk cc at 16-byte unit 8 l + (cc ^ (l & 7)); the
// bins' hi and lo parts (A operand: lane 4 q + h, head h, codewords 4 q .. 4 q + 3) accumulate into the byte
// layout's O pair 2 G, 2 G + 1 of group G.
template <int G, int CC>
__device__ __forceinline__ void wide_bin_unit(const unsigned char* vt, const int lane, const h4& ahi, const h4& alo,
                                              f4 (&O)[2 * kGroups]) {
  // the transposing read hands lane 16 q' + 4 a + e value e of the loads named by lanes 16 q' + 4 k + a: lane
  // 16 q' + 4 k + a names codeword 16 q' + 4 a + k
  const int l = (lane & 48) + 4 * (lane & 3) + ((lane >> 2) & 3);
  const unsigned char* src = vt + (8 * l + (CC ^ (l & 7))) * 16;
  const h4 v0 = lds_read_tr(src);
  const h4 v1 = lds_read_tr(src + 8);
  O[2 * G] = mfma(ahi, v0, O[2 * G]);
  O[2 * G] = mfma(alo, v0, O[2 * G]);
  O[2 * G + 1] = mfma(ahi, v1, O[2 * G + 1]);
  O[2 * G + 1] = mfma(alo, v1, O[2 * G + 1]);
}

// TAIL: residuals in the last index window, R - kRes (ceil(R / kRes) - 1), 1 .. kRes (a kernel per value, so that the
// last window's passes gather exactly its residuals).
template <int TAIL>
__global__ void __launch_bounds__(kThreads) attn_wide_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kSlot + kPhaseBytes];
  // epilogue-only LDS (placed in the codebook slots, past the reduction buffer, once the passes are done)
  auto& wave_ml = *reinterpret_cast<float(*)[2][kW][kGqa]>(lds + kW * kHeadDim * kGqa * sizeof(float));
  int& is_last = *reinterpret_cast<int*>(lds + kW * kHeadDim * kGqa * sizeof(float) + sizeof(wave_ml));

  const int kv = blockIdx.x % a.n_kv_heads, split = blockIdx.x / a.n_kv_heads, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the part of the prologue's copies this wave moves, rotated by the split: the workgroups of an XCD copy the
  // same KV head's data at the same moment and so start on different parts of it (spread over the L2 channels)
  const int part = __builtin_amdgcn_readfirstlane((wave + split) & (kW - 1));
  const int R = a.n_residuals, Wd = a.record_words;
  const int nch = (R + kRes - 1) / kRes;         // index windows
  constexpr bool tail_both = 2 * TAIL <= kRes;    // the last window in one pass over both groups
  const int npass = 2 * (nch - 1) + (tail_both ? 1 : 2);
  // (group, residual) of table t of pass p's slot (r >= R: a table of zero rows)
  auto pass_table = [&](int p, int t, int& g, int& r) {
    const int c = min(p >> 1, nch - 1);
    const bool both = tail_both && p == npass - 1;
    g = both ? (t & 1) : (p & 1);
    r = kRes * c + (both ? t >> 1 : t);
  };
  const int64_t cb_stride = static_cast<int64_t>(kWG) * R * kWN * (kWRow / 2);
  const f16* cb_k = static_cast<const f16*>(a.k_cb) + kv * cb_stride;
  const f16* cb_v = static_cast<const f16*>(a.v_cb) + kv * cb_stride;
  // sequence bounds (clamped), read before any memory operation so that they stay scalar loads
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.max_len, a.total_tokens);
  const int L = sb.len;
  const int64_t seq_start = sb.start;

  // ---------------------------------------------------------------------------------- prologue
  // A split past the end of its sequence (a ragged batch launches the longest sequence's split count for every
  // sequence) leaves at once, before any LDS copy.
  const int S = a.split_tokens;
  const int t0 = split * S;
  const int h0 = kv * kGqa;
  const int64_t bh0 = static_cast<int64_t>(b) * a.n_q_heads + h0;
  float* out_bh = a.out + bh0 * kHeadDim;
  if (t0 >= L) {
    if (split == 0)
      for (int i = tid; i < kGqa * kHeadDim; i += kThreads) out_bh[i] = 0.f;
    return;
  }
  // (1) fp32 fine phases (group-major, the byte layout's groups) and the tables of pass 0 (wave part moves
  // table part), straight into LDS.
  {
    constexpr int kFineChunks = kPhaseBytes / 16;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.rope + kRopeFine32gOffset);
#pragma unroll
    for (int i = 0; i < kFineChunks / kThreads; ++i) {
      const int c = (part * (kFineChunks / kThreads) + i) * 64;
      __builtin_amdgcn_global_load_lds(src + (c + lane) * 16, lds + kPhase + c * 16, 16, 0, 0);
    }
    static_assert(kTables == kW && kWTab / 16 == kMaxBlocks * 64, "one table per wave, 64 units per load");
    int g0, r0;
    pass_table(0, part, g0, r0);
    if (r0 < R) {
#pragma unroll
      for (int i = 0; i < kMaxBlocks; ++i) {
        const int u = i * 64 + lane;
        __builtin_amdgcn_global_load_lds(table_unit_src(cb_k, R, g0, r0, u), lds + part * kWTab + (i * 64) * 16, 16,
                                         0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kMaxBlocks; ++i)
        *reinterpret_cast<uint4*>(lds + part * kWTab + (i * 64 + lane) * 16) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const int nvalid = min(S, L - t0);
  const int nblocks = (nvalid + 63) >> 6;
  const int my_blocks = (nblocks - wave + kW - 1) / kW;
  const int64_t row_base = seq_start + t0;
  auto token_row = [&](int i) -> int64_t {
    int tl = (wave + kW * i) * 64 + lane;
    asm volatile("" : "+v"(tl));
    return row_base + min(tl, nvalid - 1);
  };

  // (2) the query pairs this lane supplies to the broadcast A operand (head lane mod 4, pairs 16 k + lane / 4)
  // and their coarse phases for the wave's first block and for row 1 (e^{i 64 theta})
  const int quad = lane >> 2, qi = lane & 3;
  const f16* qp = static_cast<const f16*>(a.q) + (bh0 + qi) * kHeadDim;
  uint32_t qraw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) qraw[k] = *reinterpret_cast<const uint32_t*>(qp + 2 * (16 * k + quad));
  const float2* coarse = a.rope + kRopeCoarseOffset;
  const int last_row = (L - 1) >> 6;
  const float2* crow0 = coarse + static_cast<int64_t>(min((t0 >> 6) + wave, last_row)) * kPairs;
  const float2* crow1 = coarse + static_cast<int64_t>(min(1, last_row)) * kPairs;
  float2 cph0[4], cph1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    cph0[k] = crow0[16 * k + quad];
    cph1[k] = crow1[16 * k + quad];
  }
  __builtin_amdgcn_sched_barrier(0);

  // (3) index words of pass 0 for every block. Step p (key passes p < npass, then value windows p - npass)
  // reads the three words of its window from their word planes: a wave's 64 tokens are 256 contiguous bytes
  // of each plane. The two key passes of a window read the same words (the second time from L2). Requests past
  // the last step read the last step's words, so every step issues the same loads (clamped rows and words,
  // always in bounds).
  const int64_t T = a.total_tokens;
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(a.k_codes) + static_cast<int64_t>(kv) * Wd * T;
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(a.v_codes) + static_cast<int64_t>(kv) * Wd * T;
  uint3 code[kMaxBlocks];
  auto request_words = [&](int pn, int i) {
    const int pc = min(pn, npass + nch - 1);
    const int c = pc < npass ? min(pc >> 1, nch - 1) : pc - npass;
    const int w0 = packed_window_word(c);
    const uint32_t* rec = (pc < npass ? kw : vw) + token_row(i);
    code[i] = make_uint3(rec[min(w0, Wd - 1) * T], rec[min(w0 + 1, Wd - 1) * T], rec[min(w0 + 2, Wd - 1) * T]);
  };
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) request_words(0, i);
  constexpr int kPrologueRecords = 3 * kMaxBlocks;

  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kPrologueRecords));
  slot_barrier();

  // A operands: q'' = q * conj(coarse phase of the block), fp32; the wave's blocks are kW rows apart, so
  // q''_{i+1} = q''_i * conj(E) with E = e^{i 64 kW theta} (row 1 squared log2(kW) times).
  float2 qc0[4], stepE[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    asm volatile("" : "+v"(qraw[k]));
    const h2 hq = as_h2(qraw[k]);
    qc0[k] = cmul_conj(make_float2(static_cast<float>(hq.x), static_cast<float>(hq.y)), cph0[k]);
    float2 e = cph1[k];
#pragma unroll
    for (int sq = 1; sq < kW; sq *= 2) e = make_float2(e.x * e.x - e.y * e.y, 2.f * e.x * e.y);
    stepE[k] = e;
  }
  const h4 ident = identity_b(lane);

  // ------------------------------------------------------------------------- key passes
  // Staging: during pass p, each thread fetches one 16-byte unit per block of pass p + 1's tables (block i:
  // table i) and writes it into slot (p + 1) % 2 one block later (that slot's last reader, pass p - 1, finished
  // at the barrier that ended it). The last pass writes zeros there instead: that slot then holds the value bins.
  uint4 stage;
  auto stage_load = [&](int pn, int i) {
    int g = 0, r = R;
    if (pn < npass) pass_table(pn, i, g, r);
    if (r < R)
      stage = *reinterpret_cast<const uint4*>(table_unit_src(cb_k, R, g, r, tid));
    else
      stage = make_uint4(0u, 0u, 0u, 0u);
  };
  auto stage_store = [&](int pn, int i) {
    *reinterpret_cast<uint4*>(lds + (pn & 1) * kSlot + (i * kThreads + tid) * 16) = stage;
  };

  f4 sc[kMaxBlocks];
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) sc[i] = (f4){0.f, 0.f, 0.f, 0.f};

  // One key pass over NR residuals of NG = kRes / NR groups of window c (NG = 1: group g, pass 2 c + g; NG = 2:
  // the last pass). Its slot holds table t = rho (NG = 1) or 2 rho + g (NG = 2) for residual kRes c + rho.
  // Units (g, cc) of the wave's blocks form one software pipeline: the gathers of unit n + kWAhead go out before
  // the arithmetic of unit n; block i + 1's row offsets are computed (and its next-pass words requested) at the
  // start of block i.
  auto key_pass = [&](auto nrc, auto ngc, const int g, const int c) {
    constexpr int NR = decltype(nrc)::value, NG = decltype(ngc)::value, NU = kChunks * NG;
    static_assert(NR * NG <= kTables, "the pass's tables fit its slot");
    const int p = NG == 1 ? 2 * c + g : npass - 1;
    const int slot_off = (p & 1) * kSlot;
    // group g's indices 2 rho + g of the window are indices 2 rho of the window shifted by 6 g
    const int sh = NG == 1 ? kWideBits * g : 0;
    const unsigned char* phases = lds + kPhase + (NG == 1 ? g * (kChunks * 2 * 64 * 16) : 0);
    uint32_t adr[2][kTables];
    uint4 rows[kWBufs][NR];
    float2 cur[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) cur[k] = qc0[k];
    auto block_addresses = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < kMaxBlocks) {
        const uint32_t x0 = __builtin_amdgcn_alignbit(code[i].y, code[i].x, sh);
        const uint32_t x1 = __builtin_amdgcn_alignbit(code[i].z, code[i].y, sh);
        const uint32_t x2 = code[i].z >> sh;
        static_for<kTables>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          const uint32_t idx = packed_index<NG == 1 ? 2 * t : t>(x0, x1, x2);
          adr[i & 1][t] = slot_off + t * kWTab + idx * kWRow + ((idx >> 1) & 7) * 16;
        });
        request_words(p + 1, i);
      }
    };
    auto issue = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NU * kMaxBlocks) {
        constexpr int i = m / NU, gu = (m % NU) / kChunks, cc = m % kChunks;
#pragma unroll
        for (int rho = 0; rho < NR; ++rho)
          rows[m % kWBufs][rho] = *reinterpret_cast<const uint4*>(lds + (adr[i & 1][NG * rho + gu] ^ (16 * cc)));
      }
    };
    block_addresses(std::integral_constant<int, 0>{});
    if (my_blocks > 0) static_for<kWAhead>(issue);
    auto block = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_s_setprio(block_prio(i));
      block_addresses(std::integral_constant<int, i + 1>{});
      if (i > 0) stage_store(p + 1, i - 1);
      stage_load(p + 1, i);
      if (i < my_blocks) {
        f4 acc[2] = {sc[i], (f4){0.f, 0.f, 0.f, 0.f}};  // real-part and imaginary-part chains
        float4 ph[2];
        // query operand pairs: byte-layout groups 8 g .. 8 g + 7 (NG = 1), all groups (NG = 2)
        const float2 cq[2] = {g ? cur[2] : cur[0], g ? cur[3] : cur[1]};
        auto unit = [&](auto uc) {
          constexpr int u = decltype(uc)::value, n = NU * i + u, cc = u % kChunks;
          constexpr int Gp = u;  // byte-layout group relative to the phase base (8 g + cc, or cc for NG = 1)
          ph[0] = *reinterpret_cast<const float4*>(phases + ((2 * Gp) * 64 + lane) * 16);
          ph[1] = *reinterpret_cast<const float4*>(phases + ((2 * Gp + 1) * 64 + lane) * 16);
          __builtin_amdgcn_sched_barrier(0);
          issue(std::integral_constant<int, n + kWAhead>{});
          __builtin_amdgcn_sched_barrier(0);
          wide_key_unit<NR, cc>(rows[n % kWBufs], ident, ph[0], ph[1], NG == 1 ? cq[cc / 4] : cur[Gp / 4], acc);
        };
        static_for<NU>(unit);
        sc[i] = acc[0] + acc[1];
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = cmul_conj(cur[k], stepE[k]);
      }
    };
    static_for<kMaxBlocks>(block);
    __builtin_amdgcn_s_setprio(0);
    stage_store(p + 1, kMaxBlocks - 1);
    lds_barrier();  // slot (p + 1) % 2 is complete; every wave is done with slot p % 2
  };

  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using Full = std::integral_constant<int, kRes>;
  using Tail = std::integral_constant<int, TAIL>;
  const int nfull = 2 * (nch - 1) + (TAIL == kRes ? 2 : 0);  // passes over full windows
  for (int p = 0; p < nfull; ++p) key_pass(Full{}, I1{}, p & 1, p >> 1);
  if constexpr (tail_both) {
    key_pass(Tail{}, I2{}, 0, nch - 1);
  } else if constexpr (TAIL < kRes) {
    key_pass(Tail{}, I1{}, 0, nch - 1);
    key_pass(Tail{}, I1{}, 1, nch - 1);
  }

  // The value tables for the bins x value codebook product below go through this wave's 8 KiB of the last key
  // pass's slot (free since that pass's closing barrier); the first one is copied now.
  constexpr int kSteps = (kWideMaxResiduals + kW - 1) / kW;
  auto step_r = [&](int g, int n) { return ((wave - g * R) % kW + kW) % kW + kW * n; };
  unsigned char* vtab = lds + ((npass - 1) & 1) * kSlot + wave * kWTab;
  auto load_vtab = [&](int g, int r) {
    const f16* tab = cb_v + (static_cast<int64_t>(g) * R + r) * kWN * (kWRow / 2);
#pragma unroll
    for (int k = 0; k < kWTab / 1024; ++k) {
      const int l = 8 * k + (lane >> 3), cc = (lane & 7) ^ (l & 7);
      __builtin_amdgcn_global_load_lds(tab + l * (kWRow / 2) + cc * 8, vtab + k * 1024, 16, 0, 0);
    }
  };
  if (step_r(0, 0) < R)
    load_vtab(0, step_r(0, 0));
  else if (step_r(1, 0) < R)
    load_vtab(1, step_r(1, 0));

  // ------------------------------------------------------------------------- softmax weights
  // M = the workgroup's maximum scaled score per head (finite: the split holds a valid token); each wave's
  // weights p = e^{s - M} in fixed point, two heads per 64-bit word; l_w = the wave's sum of them.
  float M[kGqa], l_w[kGqa];
  uint64_t fx[kMaxBlocks][2];
  {
    float* wg_m = reinterpret_cast<float*>(lds + kPhase);  // [kW][kGqa] (the phases are no longer read)
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < kMaxBlocks; ++i) {
        const bool ok = i < my_blocks && (wave + kW * i) * 64 + lane < nvalid;
        sc[i][h] = ok ? sc[i][h] * a.scale : -INFINITY;
        mx = fmaxf(mx, sc[i][h]);
      }
      mx = wave_max(mx);
      if (lane == 0) wg_m[wave * kGqa + h] = mx;
    }
    lds_barrier();
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      M[h] = wg_m[h];
#pragma unroll
      for (int w = 1; w < kW; ++w) M[h] = fmaxf(M[h], wg_m[w * kGqa + h]);
    }
    float lsum[kGqa] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      uint32_t qv[kGqa];
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        // masked tokens: e^{-inf} = 0
        qv[h] = __float2uint_rn(__expf(sc[i][h] - M[h]) * static_cast<float>(1 << kFxBits));
        lsum[h] += static_cast<float>(qv[h]);
      }
      fx[i][0] = qv[0] | (static_cast<uint64_t>(qv[1]) << 32);
      fx[i][1] = qv[2] | (static_cast<uint64_t>(qv[3]) << 32);
    }
#pragma unroll
    for (int h = 0; h < kGqa; ++h) l_w[h] = wave_sum(lsum[h]) * (1.f / static_cast<float>(1 << kFxBits));
  }

  // ------------------------------------------------------------------------- value bins
  // bins[g][r][hp][l] (64-bit words, heads 2 hp and 2 hp + 1) in the slot the last key pass zeroed. Window c
  // of every block: its 16 indices select the bins its weights go to; the words of window c + 1 are requested
  // in their place (one window ahead, as in the key passes).
  unsigned long long* bins = reinterpret_cast<unsigned long long*>(lds + (npass & 1) * kSlot);
  for (int c = 0; c < nch; ++c) {
    const int nres = min(kRes, R - kRes * c);
    auto block = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      // (every block requests its words, as in the key passes, so that the loads stay in flight)
      const uint3 w = code[i];
      request_words(npass + c + 1, i);
      if (i < my_blocks) {
        static_for<kIdx>([&](auto fc) {
          constexpr int f = decltype(fc)::value, rho = f >> 1, g = f & 1;
          if (rho < nres) {
            unsigned long long* bp = bins + ((g * R + kRes * c + rho) * 2) * kWN + packed_index<f>(w.x, w.y, w.z);
            __hip_atomic_fetch_add(bp, fx[i][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(bp + kWN, fx[i][1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        });
      }
    };
    static_for<kMaxBlocks>(block);
  }
  lds_barrier();  // every token's weights are in the bins

  // ------------------------------------------------------------------------- bins x value codebook
  // The wave takes the (g, r) of its share (every kW-th of the 2 R), in steps m = g kSteps + n with
  // r = r0(g) + kW n. Each step's value table is copied into the wave's 8 KiB of the last key pass's slot by
  // coalesced direct-to-LDS loads (codeword l's chunk cc to unit 8 l + (cc ^ (l & 7))), the next step's copy
  // going out once the current table has been read. A operand: bins of head h = lane & 3, codewords
  // 4 (lane >> 2) .. + 3, as fp16 hi + lo of their value in units of 1 (exact to 2^-22 relative).
  f4 O[2 * kGroups];
#pragma unroll
  for (int c = 0; c < 2 * kGroups; ++c) O[c] = (f4){0.f, 0.f, 0.f, 0.f};
  {
    const int hh = lane & 3, l4 = (lane >> 2) * 4;
    static_for<kWG * kSteps>([&](auto mc) {
      constexpr int m = decltype(mc)::value, g = m / kSteps, n = m % kSteps;
      const int r = step_r(g, n);
      if (r < R) {
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));  // this wave's copy of the table has landed
        const uint4* bq = reinterpret_cast<const uint4*>(bins + ((g * R + r) * 2 + (hh >> 1)) * kWN + l4);
        const uint4 u0 = bq[0], u1 = bq[1];  // codewords l4, l4 + 1 | l4 + 2, l4 + 3: (heads 2 hp, 2 hp + 1)
        const bool odd = hh & 1;
        const uint32_t cnt[4] = {odd ? u0.y : u0.x, odd ? u0.w : u0.z, odd ? u1.y : u1.x, odd ? u1.w : u1.z};
        h4 ahi, alo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const Split2 sp = split2(static_cast<float>(cnt[k]) * (1.f / static_cast<float>(1 << kFxBits)));
          ahi[k] = sp.hi;
          alo[k] = sp.lo;
        }
        static_for<kChunks>([&](auto ccc) {
          constexpr int cc = decltype(ccc)::value;
          wide_bin_unit<8 * g + cc, cc>(vtab, lane, ahi, alo, O);
        });
        __builtin_amdgcn_s_waitcnt(kLgkmcnt0);  // the table has been read: the next copy may overwrite it
        __builtin_amdgcn_sched_barrier(0);
        int gn = g, nn = n + 1;
        if (nn >= kSteps || step_r(gn, nn) >= R) {
          gn = g + 1;
          nn = 0;
        }
        if (gn < kWG && step_r(gn, nn) < R) load_vtab(gn, step_r(gn, nn));
      }
    });
  }

  // every wave's weights are relative to the same M
  float m_w[kGqa];
#pragma unroll
  for (int h = 0; h < kGqa; ++h) m_w[h] = M[h];
  attn_epilogue<kW>(a, lds, wave_ml, is_last, lane_id(), wave * 64 + lane_id(), wave, O, b, kv, split, L, S, bh0,
                    out_bh, m_w, l_w);
}

}  // namespace

hipError_t launch_attn_wide(int B, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.n_splits * a.n_kv_heads, B);
  switch (a.n_residuals - kRes * ((a.n_residuals + kRes - 1) / kRes - 1)) {
    case 1: attn_wide_kernel<1><<<grid, kThreads, 0, s>>>(a); break;
    case 2: attn_wide_kernel<2><<<grid, kThreads, 0, s>>>(a); break;
    case 3: attn_wide_kernel<3><<<grid, kThreads, 0, s>>>(a); break;
    case 4: attn_wide_kernel<4><<<grid, kThreads, 0, s>>>(a); break;
    case 5: attn_wide_kernel<5><<<grid, kThreads, 0, s>>>(a); break;
    case 6: attn_wide_kernel<6><<<grid, kThreads, 0, s>>>(a); break;
    case 7: attn_wide_kernel<7><<<grid, kThreads, 0, s>>>(a); break;
    default: attn_wide_kernel<8><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace commvq
