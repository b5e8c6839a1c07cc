// Decode-step attention over a CommVQ cache in the pages' own code shape, on gfx950.
//
// Same computation as attn_kernel (score = scale * sum_j Re(conj(q_j) khat_{t,j} e^{i t theta_j}),
// out = softmax-weighted sum of vhat), for the setting the CommVQ pages evaluate: one code index shared by
// the 64 dims of a half head (G = 2 groups of 64 dims), N = 64 codewords per residual codebook (6-bit
// indices), and many residual rounds. The average is R log2(N) / g bits per scalar (pith.science verdict
// for arXiv 2506.18879, key_machinery; its referee report's minor comments give g = 64, N' = 64), so
// R = 11 gives about 1 bit and R = 21 about 2 (the CommVQ summary page, Limitations, names these two).
// A token's R x G indices are one little-endian bitstream of 32-bit words, index (r, g) at bit 6 (r G + g).
//
// The codebooks (R x 16 KiB per KV head for keys, as much for values) do not fit in LDS, so the kernel
// runs in passes of kRes residuals: key passes c = 0 .. nch-1, then the wave softmax, then value passes.
// Pass p's codebook chunk (kRes residuals x 2 groups x 8 KiB) sits in LDS slot p % 2 while the chunk of
// pass p + 1 is staged through registers into the other slot. Scores and the value accumulators are
// linear in the residuals, so each pass adds its chunk's share to the MFMA accumulators.
//
// Work item, lanes and MFMA layouts are those of attn_kernel: lane = token of a 64-token block, 4 GQA
// heads per KV head, the per-64-token RoPE phase on the query and the per-lane phase on the keys. A
// 16-byte chunk cc of the 128-byte row of group g holds RoPE pairs 32 g + 4 cc .. + 3, exactly the pairs
// of the byte layout's group 8 g + cc, so the key MFMA step, the p^T operands, the softmax and the epilogue
// are shared. Per unit (g, cc) a lane gathers its token's chunk from each of the pass's kRes residual rows,
// sums them in fp32 on the matrix core (an MFMA with the identity as A adds a lane's four fp16 values to
// its fp32 accumulator), and then
//   keys:   rounds the sum to fp16, rotates it by the fine phase and runs the two key MFMA steps;
//   values: sums with the identity as B instead, which transposes each 4x4 (token x dim) quad tile as it
//           accumulates, then multiplies by p^T.
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
constexpr int kRes = kWideResPerPass;            // residuals per pass (4)
constexpr int kIdx = kRes * kWG;                 // indices per pass (8)
constexpr int kSlot = kIdx * kWTab;              // bytes per codebook slot (64 KiB)
constexpr int kChunks = kWRow / 16;              // 16-byte chunks per row (8)
constexpr int kUnits = kWG * kChunks;            // units (g, cc) per block (16)
constexpr int kW = 8;                            // waves per workgroup
constexpr int kThreads = kW * 64;
constexpr int kZeroRow = 2 * kSlot;              // LDS offset of a 128-byte zero row
constexpr int kWAhead = 1;                       // units whose gathers are in flight ahead of the current one
constexpr int kWBufs = kWAhead + 1;
static_assert(kSlot / 16 == kMaxBlocks * kThreads, "one staged 16-byte unit per thread per block");
static_assert(kZeroRow >= (kIdx - 1) * kWTab, "zero-row stand-in offsets stay non-negative");

// Global source of 16-byte unit u of the slot holding residuals r0 .. r0 + kRes - 1 (unit u = table
// f = 2 rho + g, codeword l, physical chunk pc). Residuals past R read residual R - 1 (never used).
__device__ __forceinline__ const unsigned char* slot_unit_src(const f16* cb_kv, int R, int r0, int u) {
  const int f = u >> 9, l = (u >> 3) & (kWN - 1), pc = u & 7;
  const int rho = f >> 1, g = f & 1;
  const int r = min(r0 + rho, R - 1);
  const int cc = pc ^ ((l >> 1) & 7);
  return reinterpret_cast<const unsigned char*>(cb_kv + ((static_cast<int64_t>(g) * R + r) * kWN + l) * (kWRow / 2)) +
         cc * 16;
}

// Sum of a unit's kRes residual chunks, in fp32 on the matrix core: with A = identity, lane 4b + j of
// D receives its own B values plus C, so k0 (dims 0..3 of the chunk) and k1 (dims 4..7) accumulate the
// lane's row chunks. The fp16 result feeds the key MFMA step of byte-layout group G.
template <int G>
__device__ __forceinline__ void wide_key_unit(const uint4 (&rows)[kRes], const h4& ident, const uint4 (&F)[kGroups],
                                              const h4& A0, const h4& A1, f4& acc) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  f4 k0 = mfma(ident, cat(as_h2(rows[0].x), as_h2(rows[0].y)), z);
  f4 k1 = mfma(ident, cat(as_h2(rows[0].z), as_h2(rows[0].w)), z);
#pragma unroll
  for (int rho = 1; rho < kRes; ++rho) {
    k0 = mfma(ident, cat(as_h2(rows[rho].x), as_h2(rows[rho].y)), k0);
    k1 = mfma(ident, cat(as_h2(rows[rho].z), as_h2(rows[rho].w)), k1);
  }
  // one v_cvt_pk_f16_f32 (round to nearest even) per pair
  auto pk = [](float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, h2));
  };
  key_step<G>(make_uint4(pk(k0[0], k0[1]), pk(k0[2], k0[3]), pk(k1[0], k1[1]), pk(k1[2], k1[3])), F, A0, A1, acc);
}

// Value unit: with B = identity, lane 4b + j of D receives value j of each lane of its quad (dim j of the
// quad's 4 tokens), so the residual sum accumulates already transposed; rounded to fp16 it is the B
// operand of p^T x v for byte-layout group G.
template <int G>
__device__ __forceinline__ void wide_value_unit(const uint4 (&rows)[kRes], const h4& ident, const h4& pt,
                                                f4 (&O)[2 * kGroups]) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  f4 x0 = mfma(cat(as_h2(rows[0].x), as_h2(rows[0].y)), ident, z);
  f4 x1 = mfma(cat(as_h2(rows[0].z), as_h2(rows[0].w)), ident, z);
#pragma unroll
  for (int rho = 1; rho < kRes; ++rho) {
    x0 = mfma(cat(as_h2(rows[rho].x), as_h2(rows[rho].y)), ident, x0);
    x1 = mfma(cat(as_h2(rows[rho].z), as_h2(rows[rho].w)), ident, x1);
  }
  O[2 * G] = mfma(pt, to_h4(x0), O[2 * G]);
  O[2 * G + 1] = mfma(pt, to_h4(x1), O[2 * G + 1]);
}

__global__ void __launch_bounds__(kThreads) attn_wide_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kSlot + kWRow];
  __shared__ __attribute__((aligned(16))) uint4 fine_lds[kGroups * kFineRows];  // packed fp16 fine phases
  __shared__ float wave_ml[2][kW][kGqa];
  __shared__ int is_last;

  const int kv = blockIdx.x % a.n_kv_heads, split = blockIdx.x / a.n_kv_heads, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.n_residuals, Wd = a.record_words;
  const int nch = (R + kRes - 1) / kRes;  // passes per kind
  const int64_t cb_stride = static_cast<int64_t>(kWG) * R * kWN * (kWRow / 2);
  const f16* cb_k = static_cast<const f16*>(a.k_cb) + kv * cb_stride;
  const f16* cb_v = static_cast<const f16*>(a.v_cb) + kv * cb_stride;
  // sequence bounds (clamped), read before any memory operation so that they stay scalar loads
  const SeqBounds sb = seq_bounds(a.seq_start, a.seq_len, b, a.max_len, a.total_tokens);
  const int L = sb.len;
  const int64_t seq_start = sb.start;

  // ---------------------------------------------------------------------------------- prologue
  // (0) the zero row that stands in for the rows of residuals past R in the last pass of each kind (an
  // ordinary store, written before any direct-to-LDS load is in flight).
  if (tid < kWRow / 16) reinterpret_cast<uint4*>(lds + kZeroRow)[tid] = make_uint4(0u, 0u, 0u, 0u);
  // (1) fine phases and the codebook chunk of pass 0 (key residuals 0 .. kRes-1), straight into LDS.
  {
    constexpr int kFineChunks = kGroups * kFineRows;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.rope + kRopeFine16Offset);
#pragma unroll
    for (int i = 0; i < kFineChunks / kThreads; ++i) {
      const int c = (wave * (kFineChunks / kThreads) + i) * 64;
      __builtin_amdgcn_global_load_lds(src + (c + lane) * 16, reinterpret_cast<unsigned char*>(fine_lds) + c * 16, 16,
                                       0, 0);
    }
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      const int u0 = wave * (kSlot / 16 / kW) + i * 64;
      __builtin_amdgcn_global_load_lds(slot_unit_src(cb_k, R, 0, u0 + lane), lds + u0 * 16, 16, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const int S = a.split_tokens;
  const int t0 = split * S;
  const int h0 = kv * kGqa;
  const int64_t bh0 = static_cast<int64_t>(b) * a.n_q_heads + h0;
  float* out_bh = a.out + bh0 * kHeadDim;
  if (t0 >= L) {
    if (split == 0)
      for (int i = tid; i < kGqa * kHeadDim; i += kThreads) out_bh[i] = 0.f;
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    return;
  }
  const int nvalid = min(S, L - t0);
  const int nblocks = (nvalid + 63) >> 6;
  const int my_blocks = (nblocks - wave + kW - 1) / kW;
  const int64_t row_base = seq_start + t0;
  auto token_row = [&](int i) -> int64_t {
    int tl = (wave + kW * i) * 64 + lane;
    asm volatile("" : "+v"(tl));
    return row_base + min(tl, nvalid - 1);
  };

  // (2) query pairs and coarse phases (rows of the wave's first block and of e^{i 64 theta})
  const int quad = lane >> 2, qi = lane & 3;
  const f16* qp = static_cast<const f16*>(a.q) + (bh0 + qi) * kHeadDim;
  uint32_t qraw[4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) qraw[2 * m + e] = *reinterpret_cast<const uint32_t*>(qp + 2 * (32 * m + 2 * quad + e));
  const float2* coarse = a.rope + kRopeCoarseOffset;
  float4 cphase[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = i == 0 ? min((t0 >> 6) + wave, (L - 1) >> 6) : min(1, (L - 1) >> 6);
#pragma unroll
    for (int m = 0; m < 2; ++m)
      cphase[i][m] = *reinterpret_cast<const float4*>(coarse + static_cast<int64_t>(row) * kPairs + 32 * m + 2 * quad);
  }
  __builtin_amdgcn_sched_barrier(0);

  // (3) index words of pass 0 for every block. Pass p reads the two words of its window (chunk c of the
  // record); requests past the last pass read the last pass's words, so every pass issues the same loads
  // (clamped rows and words, always in bounds).
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(a.k_codes);
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(a.v_codes);
  uint2 code[kMaxBlocks];
  auto request_words = [&](int pn, int i) {
    const int pc = min(pn, 2 * nch - 1);
    const int c = pc < nch ? pc : pc - nch;
    const int w0 = packed_window_word(c);
    const int w1 = min(w0 + 1, Wd - 1);
    const uint32_t* rec = (pc < nch ? kw : vw) + (static_cast<int64_t>(kv) * a.total_tokens + token_row(i)) * Wd;
    code[i] = make_uint2(rec[w0], rec[w1]);
  };
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) request_words(0, i);
  constexpr int kPrologueRecords = 2 * kMaxBlocks;

  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kPrologueRecords));
  slot_barrier();  // (its lgkmcnt(0) also retires the zero-row store before the barrier)
  uint4 F[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) F[g] = fine_lds[g * kFineRows + lane];
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(qraw[k]));
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
      asm volatile("" : "+v"(cphase[i][m].x), "+v"(cphase[i][m].y), "+v"(cphase[i][m].z), "+v"(cphase[i][m].w));

  // A operands: q'' = q * conj(coarse phase of the block); the wave's blocks are kW rows apart, so
  // q''_{i+1} = q''_i * conj(E) with E = e^{i 64 kW theta} (row 1 squared log2(kW) times).
  float2 qc0[4], stepE[4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const h2 q0 = as_h2(qraw[2 * m]), q1 = as_h2(qraw[2 * m + 1]);
    const float4 c0 = cphase[0][m], c1 = cphase[1][m];
    qc0[2 * m] = cmul_conj(make_float2(static_cast<float>(q0.x), static_cast<float>(q0.y)), make_float2(c0.x, c0.y));
    qc0[2 * m + 1] =
        cmul_conj(make_float2(static_cast<float>(q1.x), static_cast<float>(q1.y)), make_float2(c0.z, c0.w));
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
  const h4 ident = identity_b(lane);

  // ------------------------------------------------------------------------- pass machinery
  // Staging: during pass p, each thread fetches one 16-byte unit per block of pass p + 1's codebook chunk
  // and writes it into slot (p + 1) % 2 one block later (that slot's last reader, pass p - 1, finished at
  // the barrier that ended it).
  uint4 stage;
  auto stage_src = [&](int pn, int i) {
    const int pc = min(pn, 2 * nch - 1);
    const bool key = pc < nch;
    return slot_unit_src(key ? cb_k : cb_v, R, kRes * (key ? pc : pc - nch), i * kThreads + tid);
  };
  auto stage_load = [&](int pn, int i) { stage = *reinterpret_cast<const uint4*>(stage_src(pn, i)); };
  auto stage_store = [&](int pn, int i) {
    *reinterpret_cast<uint4*>(lds + (pn & 1) * kSlot + (i * kThreads + tid) * 16) = stage;
  };
  // LDS offsets (without the table offset f * kWTab) of the rows of a block's kIdx indices in pass p.
  auto addresses = [&](int c, int slot_off, int nres, const uint2 w, uint32_t (&adr)[kIdx]) {
    uint32_t x0, x1;
    packed_window(w.x, w.y, packed_window_shift(c), x0, x1);
    static_for<kIdx>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      const uint32_t idx = packed_index<f>(x0, x1);
      const uint32_t real = slot_off + idx * kWRow + ((idx >> 1) & 7) * 16;
      adr[f] = (f >> 1) < nres ? real : static_cast<uint32_t>(kZeroRow - f * kWTab);
    });
  };

  f4 sc[kMaxBlocks];
#pragma unroll
  for (int i = 0; i < kMaxBlocks; ++i) sc[i] = (f4){0.f, 0.f, 0.f, 0.f};
  f4 O[2 * kGroups];  // value accumulators (zeroed after the key passes)
  h4 pth[kMaxBlocks];

  // One pass: kind 0 = keys (chunk c, pass p = c), kind 1 = values (pass p = nch + c). Units (g, cc) of
  // the wave's blocks form one software pipeline: the gathers of unit n + kWAhead go out before the
  // arithmetic of unit n; block i + 1's row offsets are computed (and its next-pass words requested) at
  // the start of block i.
  auto pass = [&](auto kind_c, const int c) {
    constexpr bool kKey = decltype(kind_c)::value == 0;
    const int p = kKey ? c : nch + c;
    const int slot_off = (p & 1) * kSlot;
    const int nres = min(kRes, R - kRes * c);
    uint32_t adr[2][kIdx];
    uint4 rows[kWBufs][kRes];
    float2 cur[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) cur[k] = qc0[k];
    auto block_addresses = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < kMaxBlocks) {
        addresses(c, slot_off, nres, code[i], adr[i & 1]);
        request_words(p + 1, i);
      }
    };
    auto issue = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < kUnits * kMaxBlocks) {
        constexpr int i = m / kUnits, u = m % kUnits, g = u / kChunks, cc = u % kChunks;
#pragma unroll
        for (int rho = 0; rho < kRes; ++rho)
          rows[m % kWBufs][rho] =
              *reinterpret_cast<const uint4*>(lds + (adr[i & 1][2 * rho + g] ^ (16 * cc)) + (2 * rho + g) * kWTab);
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
        if constexpr (kKey) {
          const h4 A0 = {(f16)cur[0].x, (f16)cur[0].y, (f16)cur[1].x, (f16)cur[1].y};
          const h4 A1 = {(f16)cur[2].x, (f16)cur[2].y, (f16)cur[3].x, (f16)cur[3].y};
          f4 odd = {0.f, 0.f, 0.f, 0.f};
          auto unit = [&](auto uc) {
            constexpr int u = decltype(uc)::value, n = kUnits * i + u;
            constexpr int G = (u / kChunks) * 8 + u % kChunks;  // byte-layout group of (g, cc)
            __builtin_amdgcn_sched_barrier(0);
            issue(std::integral_constant<int, n + kWAhead>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (u % 2 == 0) {
              wide_key_unit<G>(rows[n % kWBufs], ident, F, A0, A1, sc[i]);
            } else {
              wide_key_unit<G>(rows[n % kWBufs], ident, F, A0, A1, odd);
            }
          };
          static_for<kUnits>(unit);
          sc[i] += odd;
#pragma unroll
          for (int k = 0; k < 4; ++k) cur[k] = cmul_conj(cur[k], stepE[k]);
        } else {
          auto unit = [&](auto uc) {
            constexpr int u = decltype(uc)::value, n = kUnits * i + u;
            constexpr int G = (u / kChunks) * 8 + u % kChunks;
            __builtin_amdgcn_sched_barrier(0);
            issue(std::integral_constant<int, n + kWAhead>{});
            __builtin_amdgcn_sched_barrier(0);
            wide_value_unit<G>(rows[n % kWBufs], ident, pth[i], O);
          };
          static_for<kUnits>(unit);
        }
      }
    };
    static_for<kMaxBlocks>(block);
    __builtin_amdgcn_s_setprio(0);
    stage_store(p + 1, kMaxBlocks - 1);
    lds_barrier();  // pass p + 1's chunk is complete; every wave is done with slot p % 2
  };

  for (int c = 0; c < nch; ++c) pass(std::integral_constant<int, 0>{}, c);

  wave_softmax<kW>(sc, my_blocks, wave, lane, nvalid, a.scale, wave_ml);
  {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) pth[i] = to_h4(mfma(to_h4(sc[i]), ident, z));  // quad transpose of p
  }

#pragma unroll
  for (int c = 0; c < 2 * kGroups; ++c) O[c] = (f4){0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) pass(std::integral_constant<int, 1>{}, c);

  attn_epilogue<kW>(a, lds, wave_ml, is_last, lane_id(), wave * 64 + lane_id(), wave, O, b, kv, split, L, S, bh0,
                    out_bh);
}

}  // namespace

hipError_t launch_attn_wide(int B, const AttnArgs& a, hipStream_t s) {
  attn_wide_kernel<<<dim3(a.n_splits * a.n_kv_heads, B), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace commvq
