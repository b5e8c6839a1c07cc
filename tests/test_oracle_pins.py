"""Pins of the fp64 oracle to things other than itself (CPU only).

Which pin covers which oracle function:
  oracle_key_block / oracle_rotation : commutation identity R C == C R per 2x2 block; C e1 == (a, b)
  oracle_rope       : agreement with a complex-exponential formulation; group law rope(rope(x,a),b) ==
                      rope(x,a+b); norm preservation; identity at position 0; the frequency ladder
                      theta_0 = 1 and a constant ratio base^(-2/D) between neighbouring pairs
  oracle_decode     : one-hot "counting" codebooks reveal every stored index (layout pin); numpy
                      gather-and-sum on random data
  oracle_unpack     : a closed-form byte pattern comes back exactly
  oracle_table      : closed forms for q = e_{2j} (T = (a, b)) and q = e_{2j+1} (T = (b, -a))
  oracle_scores_via_table vs scores of oracle_attn_decode : the table-gather score equals the
                      decode-then-dot score to 1e-12 (the two formulations the pages relate)
  oracle_attn_decode: softmax rows sum to 1 and log-ratios equal score differences; L = 1 gives the
                      decoded value; q = 0 gives the code-histogram mean (closed form); a hand-worked
                      D = 4 example; torch's scaled_dot_product_attention in fp64 over explicitly
                      decoded keys rotated with complex exponentials; shifting every value by a constant
                      shifts the output by it; GQA mapping and ragged batches agree with per-head /
                      per-sequence runs
  oracle_value_reduce: binning identity against p @ (explicitly decoded values) to 1e-12; one-hot p
                      selects one decoded value
  oracle_encode_greedy: exact codewords are recovered; brute force over all codes for R = 1;
                      ties go to the lowest index; residual rounds never increase the error
  oracle_encode_eval: numpy brute force of the replayed rounds for arbitrary given codes; on the
                      greedy encoder's own codes the chosen distance is the minimum
Page figures (tests/golden/page_figures.json): bit-rate and memory arithmetic of the layouts.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def small_inputs(B=1, Hq=4, Hkv=1, lengths=(37,), R=2, D=16, G=2, N=16, seed=0, base=10000.0):
    rng = np.random.default_rng(seed)
    W = D // G
    seq_len = np.asarray(lengths, dtype=np.int32)
    seq_start = np.concatenate([[0], np.cumsum(seq_len[:-1])]).astype(np.int64)
    T = int(seq_len.sum())
    d = oracle.dims(B, Hq, Hkv, R, head_dim=D, n_groups=G, n_codes=N, rope_base=base)
    q = rng.standard_normal((B, Hq, D))
    kcb = rng.standard_normal((Hkv, G, R, N, W)) * 0.5
    vcb = rng.standard_normal((Hkv, G, R, N, W)) * 0.5
    kc = rng.integers(0, N, size=(Hkv, R, T, G)).astype(np.uint8)
    vc = rng.integers(0, N, size=(Hkv, R, T, G)).astype(np.uint8)
    return d, q, kcb, vcb, kc, vc, seq_start, seq_len


# ----------------------------------------------------------------------------------- blocks, RoPE
def test_commutation_identity_per_block(oracle_lib):
    rng = np.random.default_rng(1)
    for _ in range(200):
        a, b = rng.standard_normal(2)
        phi = rng.uniform(-1e4, 1e4)
        C, Rm = oracle.key_block(a, b), oracle.rotation(phi)
        assert np.max(np.abs(Rm @ C - C @ Rm)) <= 1e-15 * (1 + abs(a) + abs(b)) * 4
        np.testing.assert_array_equal(C @ np.array([1.0, 0.0]), [a, b])
        # rotation is orthogonal with determinant 1
        assert abs(np.linalg.det(Rm) - 1.0) < 1e-14
    # a matrix that is not of the block form does not commute (the identity is not vacuous)
    M = np.array([[1.0, 2.0], [3.0, 4.0]])
    Rm = oracle.rotation(0.7)
    assert np.max(np.abs(Rm @ M - M @ Rm)) > 0.1


def test_rope_matches_complex_exponential(oracle_lib):
    D, base = 128, 500000.0
    d = oracle.dims(1, 1, 1, 1, head_dim=D, rope_base=base)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, D))
    pos = rng.integers(0, 200000, size=50)
    out = oracle.rope(d, x, pos)
    theta = base ** (-np.arange(D // 2) * 2.0 / D)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * np.outer(pos, theta))
    np.testing.assert_allclose(out[:, 0::2], z.real, atol=1e-12)
    np.testing.assert_allclose(out[:, 1::2], z.imag, atol=1e-12)


def test_rope_group_law_norm_identity_and_ladder(oracle_lib):
    D = 128
    d = oracle.dims(1, 1, 1, 1, head_dim=D, rope_base=500000.0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, D))
    a = rng.integers(0, 70000, size=20)
    b = rng.integers(0, 70000, size=20)
    two = oracle.rope(d, oracle.rope(d, x, a), b)
    one = oracle.rope(d, x, a + b)
    np.testing.assert_allclose(two, one, atol=1e-10)
    pn = lambda v: v[:, 0::2] ** 2 + v[:, 1::2] ** 2
    np.testing.assert_allclose(pn(oracle.rope(d, x, a)), pn(x), rtol=1e-13)
    np.testing.assert_array_equal(oracle.rope(d, x, np.zeros(20, dtype=np.int64)), x)
    # frequency ladder: rotate e_{2j} by position 1 and read the angle back
    E = np.zeros((D // 2, D))
    E[np.arange(D // 2), 2 * np.arange(D // 2)] = 1.0
    r = oracle.rope(d, E, np.ones(D // 2, dtype=np.int64))
    ang = np.arctan2(r[np.arange(D // 2), 2 * np.arange(D // 2) + 1], r[np.arange(D // 2), 2 * np.arange(D // 2)])
    assert abs(ang[0] - 1.0) < 1e-15  # theta_0 = base^0 = 1 radian per position
    ratio = ang[1:] / ang[:-1]
    np.testing.assert_allclose(ratio, 500000.0 ** (-2.0 / D), rtol=1e-12)


# --------------------------------------------------------------------------------- unpack, decode
def test_unpack_closed_form_pattern(oracle_lib):
    d = oracle.dims(1, 4, 3, 2)
    T = 70
    kv, r, t, g = np.meshgrid(np.arange(3), np.arange(2), np.arange(T), np.arange(16), indexing="ij")
    pat = ((kv * 7 + t * 3 + r * 5 + g * 11) % 256).astype(np.uint8)
    out = oracle.unpack(d, pat, T)
    assert out.dtype == np.int32
    np.testing.assert_array_equal(out, (kv * 7 + t * 3 + r * 5 + g * 11) % 256)


def test_decode_counting_codebook_reveals_indices(oracle_lib):
    # codeword (kv, g, r, l) = l * 256^r in every dim: the decoded group value is sum_r i_r * 256^r,
    # an exact integer from which every index is read back
    Hkv, G, R, N, D = 2, 16, 2, 256, 128
    W = D // G
    d = oracle.dims(1, 4, Hkv, R)
    cb = np.zeros((Hkv, G, R, N, W))
    for r in range(R):
        cb[:, :, r, :, :] = (np.arange(N) * 256.0 ** r)[None, None, :, None]
    rng = np.random.default_rng(4)
    T = 33
    codes = rng.integers(0, 256, size=(Hkv, R, T, G)).astype(np.uint8)
    dec = oracle.decode(d, cb, codes, T)  # [Hkv][T][D]
    val = dec.reshape(Hkv, T, G, W)
    assert np.all(val == val[..., :1])
    v = val[..., 0].astype(np.int64)
    np.testing.assert_array_equal(v % 256, codes[:, 0, :, :])
    np.testing.assert_array_equal(v // 256, codes[:, 1, :, :])


def test_decode_matches_numpy_gather(oracle_lib):
    d, q, kcb, vcb, kc, vc, ss, sl = small_inputs(Hkv=2, Hq=8, lengths=(41,), R=3)
    T = kc.shape[2]
    dec = oracle.decode(d, vcb, vc, T)
    Hkv, G, R, N, W = vcb.shape
    ref = np.zeros((Hkv, T, G, W))
    for r in range(R):
        ref += vcb[np.arange(Hkv)[:, None, None], np.arange(G)[None, None, :], r, vc[:, r, :, :]]
    np.testing.assert_allclose(dec, ref.reshape(Hkv, T, G * W), atol=1e-14)


# ---------------------------------------------------------------------------------- table, scores
def test_table_closed_forms(oracle_lib):
    B, Hq, Hkv, R, D = 1, 2, 1, 2, 128
    d = oracle.dims(B, Hq, Hkv, R)
    rng = np.random.default_rng(5)
    kcb = rng.standard_normal((Hkv, 16, R, 256, 8))
    j = 21  # pair 21 lies in group 5, slot 1
    q = np.zeros((B, Hq, D))
    q[0, 0, 2 * j] = 1.0       # q_j = 1
    q[0, 1, 2 * j + 1] = 1.0   # q_j = i
    T = oracle.table(d, q, kcb)  # [B][Hq][G][R][N][W]
    g, u = divmod(j, 4)
    a, b = kcb[0, g, :, :, 2 * u], kcb[0, g, :, :, 2 * u + 1]
    np.testing.assert_array_equal(T[0, 0, g, :, :, 2 * u], a)
    np.testing.assert_array_equal(T[0, 0, g, :, :, 2 * u + 1], b)
    np.testing.assert_array_equal(T[0, 1, g, :, :, 2 * u], b)
    np.testing.assert_array_equal(T[0, 1, g, :, :, 2 * u + 1], -a)
    # every other pair sees q_j = 0
    mask = np.ones((16, 4), dtype=bool)
    mask[g, u] = False
    Tp = T[0, 0].reshape(16, R, 256, 4, 2).transpose(0, 3, 1, 2, 4)
    assert np.all(Tp[mask] == 0.0)


@pytest.mark.parametrize("R", [1, 2])
def test_table_score_equals_decode_then_dot(oracle_lib, R):
    cfg = workloads.custom("pin", 2, 8, 2, (300, 129), R, "float32", 11)
    inp = workloads.make_inputs(cfg)
    d = oracle.dims_of(cfg)
    L = int(inp["max_len"])
    _, s_ref, _ = oracle.attn_decode(d, inp["q"], inp["k_codes"], inp["v_codes"], inp["k_cb"], inp["v_cb"],
                                     inp["seq_start"], inp["seq_len"], L, want_scores=True)
    T = oracle.table(d, inp["q"], inp["k_cb"])
    s_tab = oracle.scores_via_table(d, T, inp["k_codes"], inp["seq_start"], inp["seq_len"], L)
    scale = np.abs(s_ref).max()
    assert np.max(np.abs(s_tab - s_ref)) <= 1e-12 * scale


# --------------------------------------------------------------------------------- full attention
def test_softmax_rows_sum_to_one_and_log_ratios(oracle_lib):
    cfg = workloads.custom("pin", 3, 8, 2, (1, 77, 500), 2, "float32", 12)
    inp = workloads.make_inputs(cfg)
    d = oracle.dims_of(cfg)
    L = int(inp["max_len"])
    _, s, p = oracle.attn_decode(d, inp["q"], inp["k_codes"], inp["v_codes"], inp["k_cb"], inp["v_cb"],
                                 inp["seq_start"], inp["seq_len"], L, want_scores=True, want_p=True)
    for b, lb in enumerate(inp["seq_len"]):
        ps = p[b, :, :lb]
        assert np.all(ps > 0)
        np.testing.assert_allclose(ps.sum(-1), 1.0, atol=1e-12)
        np.testing.assert_allclose(np.log(ps) - np.log(ps[:, :1]), s[b, :, :lb] - s[b, :, :1], atol=1e-10)
        assert np.all(p[b, :, lb:] == 0)


def test_single_token_returns_its_decoded_value(oracle_lib):
    d, q, kcb, vcb, kc, vc, ss, sl = small_inputs(Hq=4, Hkv=1, lengths=(1,), R=2, D=128, G=16, N=256, seed=6)
    out = oracle.attn_decode(d, q, kc, vc, kcb, vcb, ss, sl)
    v0 = sum(vcb[0, np.arange(16), r, vc[0, r, 0, :]] for r in range(2)).reshape(128)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v0, atol=1e-15)


def test_zero_query_gives_histogram_mean(oracle_lib):
    d, q, kcb, vcb, kc, vc, ss, sl = small_inputs(Hq=4, Hkv=1, lengths=(1000,), R=2, D=128, G=16, N=256, seed=7)
    q[:] = 0.0
    out = oracle.attn_decode(d, q, kc, vc, kcb, vcb, ss, sl)
    L = 1000
    ref = np.zeros((16, 8))
    for g in range(16):
        for r in range(2):
            cnt = np.bincount(vc[0, r, :, g], minlength=256)
            ref[g] += cnt @ vcb[0, g, r] / L
    for h in range(4):
        np.testing.assert_allclose(out[0, h], ref.reshape(128), atol=1e-14)


def test_hand_worked_two_token_example(oracle_lib):
    # D = 4 (two RoPE pairs), one group of 4 dims, R = 1, N = 2, one q head, L = 2, scale 1/2.
    # key codewords: l=0 -> pairs (1,0),(0,1); l=1 -> pairs (0,1),(1,0); keys use codes 0 then 1.
    # q = (1, 0, 0, 0). Token 0 (position 0, no rotation): q.k = 1 -> s0 = 1/2.
    # Token 1 (position 1): pair 0 (0,1) rotated by theta_0 * 1 = 1 rad -> (-sin 1, cos 1),
    # so q.k = -sin(1) -> s1 = -sin(1)/2. Values: l=0 -> (1,2,3,4), l=1 -> (5,6,7,8).
    d = oracle.dims(1, 1, 1, 1, head_dim=4, n_groups=1, n_codes=2, rope_base=10000.0, softmax_scale=0.5)
    kcb = np.array([[1, 0, 0, 1], [0, 1, 1, 0]], dtype=np.float64).reshape(1, 1, 1, 2, 4)
    vcb = np.array([[1, 2, 3, 4], [5, 6, 7, 8]], dtype=np.float64).reshape(1, 1, 1, 2, 4)
    kc = np.array([0, 1], dtype=np.uint8).reshape(1, 1, 2, 1)
    vc = np.array([0, 1], dtype=np.uint8).reshape(1, 1, 2, 1)
    q = np.array([1, 0, 0, 0], dtype=np.float64).reshape(1, 1, 4)
    out = oracle.attn_decode(d, q, kc, vc, kcb, vcb, np.array([0]), np.array([2], dtype=np.int32))
    s0, s1 = 0.5, -math.sin(1.0) / 2
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    ref = p0 * np.array([1, 2, 3, 4]) + (1 - p0) * np.array([5, 6, 7, 8])
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-15)


def test_matches_torch_sdpa_over_explicit_keys(oracle_lib):
    torch = pytest.importorskip("torch")
    cfg = workloads.custom("pin", 1, 8, 2, (700,), 2, "float16", 13)
    inp = workloads.make_inputs(cfg)
    d = oracle.dims_of(cfg)
    out = oracle.run_config(cfg, inp)
    q = inp["q"].astype(np.float64)
    kcb, vcb = inp["k_cb"].astype(np.float64), inp["v_cb"].astype(np.float64)
    kc, vc = inp["k_codes"], inp["v_codes"]
    L = 700
    theta = cfg.rope_base ** (-np.arange(64) * 2.0 / 128)
    ph = np.exp(1j * np.outer(np.arange(L), theta))
    for kv in range(2):
        K = sum(kcb[kv, np.arange(16)[None, :], r, kc[kv, r, :, :]] for r in range(2)).reshape(L, 128)
        V = sum(vcb[kv, np.arange(16)[None, :], r, vc[kv, r, :, :]] for r in range(2)).reshape(L, 128)
        Kc = (K[:, 0::2] + 1j * K[:, 1::2]) * ph
        Kr = np.empty_like(K)
        Kr[:, 0::2], Kr[:, 1::2] = Kc.real, Kc.imag
        Q = torch.from_numpy(q[0, 4 * kv:4 * kv + 4])[:, None, :]          # [4][1][D]
        Kt = torch.from_numpy(Kr)[None].expand(4, L, 128).contiguous()
        Vt = torch.from_numpy(V)[None].expand(4, L, 128).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, scale=cfg.softmax_scale)[:, 0]
        np.testing.assert_allclose(out[0, 4 * kv:4 * kv + 4], ref.numpy(), atol=1e-12)


def test_value_shift_equivariance(oracle_lib):
    d, q, kcb, vcb, kc, vc, ss, sl = small_inputs(Hq=4, Hkv=1, lengths=(200,), R=2, D=128, G=16, N=256, seed=8)
    out = oracle.attn_decode(d, q, kc, vc, kcb, vcb, ss, sl)
    c = np.linspace(-1, 1, 128).reshape(16, 8)
    vcb2 = vcb.copy()
    vcb2[0, :, 0, :, :] += c[:, None, :]
    out2 = oracle.attn_decode(d, q, kc, vc, kcb, vcb2, ss, sl)
    np.testing.assert_allclose(out2 - out, np.broadcast_to(c.reshape(128), out.shape), atol=1e-13)


def test_gqa_and_ragged_match_separate_runs(oracle_lib):
    cfg = workloads.custom("pin", 3, 8, 2, (50, 1, 90), 2, "float32", 14)
    inp = workloads.make_inputs(cfg)
    d = oracle.dims_of(cfg)
    full = oracle.run_config(cfg, inp)
    for b in range(3):
        s0, L = int(inp["seq_start"][b]), int(inp["seq_len"][b])
        for kv in range(2):
            d1 = oracle.dims(1, 4, 1, 2)
            out = oracle.attn_decode(d1, inp["q"][b:b + 1, 4 * kv:4 * kv + 4], inp["k_codes"][kv:kv + 1, :, s0:s0 + L],
                                     inp["v_codes"][kv:kv + 1, :, s0:s0 + L], inp["k_cb"][kv:kv + 1],
                                     inp["v_cb"][kv:kv + 1], np.array([0]), np.array([L], dtype=np.int32))
            np.testing.assert_array_equal(out[0], full[b, 4 * kv:4 * kv + 4])


def test_brute_force_loops_tiny(oracle_lib):
    d, q, kcb, vcb, kc, vc, ss, sl = small_inputs(B=1, Hq=2, Hkv=1, lengths=(6,), R=2, D=8, G=2, N=5, seed=9,
                                                  base=100.0)
    out = oracle.attn_decode(d, q, kc, vc, kcb, vcb, ss, sl)
    D, G, W = 8, 2, 4
    for h in range(2):
        s = []
        for t in range(6):
            k = [0.0] * D
            for g in range(G):
                for r in range(2):
                    for w in range(W):
                        k[g * W + w] += kcb[0, g, r, kc[0, r, t, g], w]
            acc = 0.0
            for j in range(D // 2):
                ang = t * 100.0 ** (-2.0 * j / D)
                x0 = k[2 * j] * math.cos(ang) - k[2 * j + 1] * math.sin(ang)
                x1 = k[2 * j] * math.sin(ang) + k[2 * j + 1] * math.cos(ang)
                acc += q[0, h, 2 * j] * x0 + q[0, h, 2 * j + 1] * x1
            s.append(acc / math.sqrt(D))
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        o = [0.0] * D
        for t in range(6):
            for g in range(G):
                for r in range(2):
                    for w in range(W):
                        o[g * W + w] += e[t] / z * vcb[0, g, r, vc[0, r, t, g], w]
        np.testing.assert_allclose(out[0, h], o, atol=1e-14)


# ----------------------------------------------------------------------------------- value reduce
def test_value_binning_identity(oracle_lib):
    cfg = workloads.custom("pin", 2, 8, 2, (333, 64), 2, "float16", 15)
    inp = workloads.make_inputs(cfg)
    d = oracle.dims_of(cfg)
    L = int(inp["max_len"])
    rng = np.random.default_rng(16)
    p = rng.uniform(0, 1, size=(2, 8, L))
    out = oracle.value_reduce(d, p, inp["v_codes"], inp["v_cb"], inp["seq_start"], inp["seq_len"], L)
    dec = oracle.decode(d, inp["v_cb"], inp["v_codes"], int(inp["total_tokens"]))
    for b in range(2):
        s0, lb = int(inp["seq_start"][b]), int(inp["seq_len"][b])
        for h in range(8):
            ref = p[b, h, :lb] @ dec[h // 4, s0:s0 + lb]
            assert np.max(np.abs(out[b, h] - ref)) <= 1e-12 * np.abs(ref).max()


def test_value_binning_identity_bit_packed_shape(oracle_lib):
    """The same identity at the pages' own shape (one index per 64 dims, N = 64, R = 11), codes read from
    bit-packed records."""
    cfg = workloads.custom("pin", 2, 8, 2, (333, 64), 11, "float16", 18, n_groups=2, n_codes=64)
    inp = workloads.make_inputs(cfg)
    d = oracle.dims_of(cfg)
    T, L = int(inp["total_tokens"]), int(inp["max_len"])
    vc = oracle.unpack_bits(d, inp["v_codes"], T)
    rng = np.random.default_rng(19)
    p = rng.uniform(-1, 1, size=(2, 8, L))
    out = oracle.value_reduce(d, p, vc, inp["v_cb"], inp["seq_start"], inp["seq_len"], L)
    dec = oracle.decode(d, inp["v_cb"], vc, T)
    for b in range(2):
        s0, lb = int(inp["seq_start"][b]), int(inp["seq_len"][b])
        for h in range(8):
            ref = p[b, h, :lb] @ dec[h // 4, s0:s0 + lb]
            assert np.max(np.abs(out[b, h] - ref)) <= 1e-12 * np.abs(ref).max()


def test_table_closed_forms_bit_packed_shape(oracle_lib):
    """A one-hot query picks out one RoPE pair of the 64-dim groups: q_j = 1 gives (a, b), q_j = i gives (b, -a)."""
    B, Hq, Hkv, R, D = 1, 2, 1, 3, 128
    d = oracle.dims(B, Hq, Hkv, R, n_groups=2, n_codes=64)
    rng = np.random.default_rng(6)
    kcb = rng.standard_normal((Hkv, 2, R, 64, 64))
    j = 45  # pair 45 lies in group 1, slot 13
    q = np.zeros((B, Hq, D))
    q[0, 0, 2 * j] = 1.0
    q[0, 1, 2 * j + 1] = 1.0
    T = oracle.table(d, q, kcb)  # [B][Hq][2][R][64][64]
    g, u = divmod(j, 32)
    a, b = kcb[0, g, :, :, 2 * u], kcb[0, g, :, :, 2 * u + 1]
    np.testing.assert_array_equal(T[0, 0, g, :, :, 2 * u], a)
    np.testing.assert_array_equal(T[0, 0, g, :, :, 2 * u + 1], b)
    np.testing.assert_array_equal(T[0, 1, g, :, :, 2 * u], b)
    np.testing.assert_array_equal(T[0, 1, g, :, :, 2 * u + 1], -a)
    mask = np.ones((2, 32), dtype=bool)
    mask[g, u] = False
    Tp = T[0, 0].reshape(2, R, 64, 32, 2).transpose(0, 3, 1, 2, 4)
    assert np.all(Tp[mask] == 0.0)


def test_value_reduce_one_hot_selects_token(oracle_lib):
    cfg = workloads.custom("pin", 1, 4, 1, (90,), 1, "float32", 17)
    inp = workloads.make_inputs(cfg)
    d = oracle.dims_of(cfg)
    p = np.zeros((1, 4, 90))
    p[0, np.arange(4), [0, 5, 44, 89]] = 1.0
    out = oracle.value_reduce(d, p, inp["v_codes"], inp["v_cb"], inp["seq_start"], inp["seq_len"], 90)
    dec = oracle.decode(d, inp["v_cb"], inp["v_codes"], 90)
    for h, t in enumerate([0, 5, 44, 89]):
        np.testing.assert_array_equal(out[0, h], dec[0, t])


# ---------------------------------------------------------------------------------------- encoder
def test_encode_recovers_exact_codewords(oracle_lib):
    rng = np.random.default_rng(18)
    d = oracle.dims(1, 4, 2, 1)
    cb = rng.standard_normal((2, 16, 1, 256, 8))
    codes = rng.integers(0, 256, size=(2, 1, 40, 16)).astype(np.uint8)
    x = oracle.decode(d, cb, codes, 40)
    got, dist = oracle.encode_greedy(d, x, cb, want_dist=True)
    np.testing.assert_array_equal(got, codes)
    assert np.all(dist == 0.0)


def test_encode_brute_force_and_ties(oracle_lib):
    rng = np.random.default_rng(19)
    d = oracle.dims(1, 4, 1, 1)
    cb = rng.standard_normal((1, 16, 1, 256, 8))
    cb[0, 3, 0, 200] = cb[0, 3, 0, 17]  # duplicate row: ties must go to 17
    x = rng.standard_normal((1, 30, 128))
    x[0, 0, 24:32] = cb[0, 3, 0, 17]
    got, dist = oracle.encode_greedy(d, x, cb, want_dist=True)
    for t in range(30):
        for g in range(16):
            dd = ((x[0, t, g * 8:(g + 1) * 8][None, :] - cb[0, g, 0]) ** 2).sum(-1)
            assert got[0, 0, t, g] == int(np.argmin(dd))
            assert dist[0, 0, t, g] == pytest.approx(dd.min(), rel=1e-12, abs=1e-15)
    assert got[0, 0, 0, 3] == 17


def test_encode_residual_rounds_do_not_increase_error(oracle_lib):
    rng = np.random.default_rng(20)
    d = oracle.dims(1, 4, 1, 3)
    cb = rng.standard_normal((1, 16, 3, 256, 8)) * np.array([0.5, 0.25, 0.125])[None, None, :, None, None]
    x = rng.standard_normal((1, 25, 128)) * 0.5
    codes, dist = oracle.encode_greedy(d, x, cb, want_dist=True)
    assert np.all(np.diff(dist, axis=1) <= 1e-15)
    # the last round's distance is the squared error of the decoded reconstruction
    rec = oracle.decode(d, cb, codes, 25)
    err = ((x - rec) ** 2).reshape(1, 25, 16, 8).sum(-1)
    np.testing.assert_allclose(dist[:, 2, :, :], err, rtol=1e-10, atol=1e-14)


def test_encode_eval_brute_force_and_greedy_consistency(oracle_lib):
    rng = np.random.default_rng(21)
    Hkv, R, n, G, N, W = 2, 2, 9, 16, 256, 8
    d = oracle.dims(1, 4, Hkv, R)
    cb = rng.standard_normal((Hkv, G, R, N, W)) * 0.5
    x = rng.standard_normal((Hkv, n, G * W)) * 0.7
    given = rng.integers(0, N, size=(Hkv, R, n, G)).astype(np.uint8)
    chosen, best, second = oracle.encode_eval(d, x, cb, given)
    for kv in range(Hkv):
        for t in range(n):
            for g in range(G):
                res = x[kv, t, g * W:(g + 1) * W].copy()
                for r in range(R):
                    dd = ((res[None, :] - cb[kv, g, r]) ** 2).sum(-1)
                    srt = np.sort(dd)
                    l = given[kv, r, t, g]
                    assert chosen[kv, r, t, g] == pytest.approx(dd[l], rel=1e-13)
                    assert best[kv, r, t, g] == pytest.approx(srt[0], rel=1e-13)
                    assert second[kv, r, t, g] == pytest.approx(srt[1], rel=1e-13)
                    res -= cb[kv, g, r, l]
    codes, dist = oracle.encode_greedy(d, x, cb, want_dist=True)
    chosen, best, _ = oracle.encode_eval(d, x, cb, codes)
    np.testing.assert_array_equal(chosen, best)
    np.testing.assert_array_equal(best, dist)


# ------------------------------------------------------------------------- bit-packed indices (g = 64)
def _pack_bits_bigint(idx, bits):
    """Reference packing from the definition of a little-endian bitstream: one Python integer per token,
    index k (k = r*G + g) at bit offset bits*k, cut into 32-bit words; word w of token t goes to [kv][w][t]."""
    Hkv, R, T, G = idx.shape
    nwords = (bits * R * G + 31) // 32
    out = np.zeros((Hkv, nwords, T), dtype=np.uint32)
    for kv in range(Hkv):
        for t in range(T):
            v = 0
            for r in range(R):
                for g in range(G):
                    v |= int(idx[kv, r, t, g]) << (bits * (r * G + g))
            for k in range(nwords):
                out[kv, k, t] = (v >> (32 * k)) & 0xFFFFFFFF
    return out


@pytest.mark.parametrize("R,G,N", [(11, 2, 64), (21, 2, 64), (3, 4, 16), (5, 2, 128)])
def test_unpack_bits_matches_bigint_stream(oracle_lib, R, G, N):
    rng = np.random.default_rng(40 + R)
    d = oracle.dims(1, 4, 2, R, head_dim=64 * G, n_groups=G, n_codes=N)
    idx = rng.integers(0, N, size=(2, R, 7, G)).astype(np.uint8)
    bits = int(np.log2(N))
    np.testing.assert_array_equal(oracle.unpack_bits(d, _pack_bits_bigint(idx, bits), 7), idx)


def test_unpack_bits_hand_worked_words(oracle_lib):
    d = oracle.dims(1, 4, 1, 11, head_dim=128, n_groups=2, n_codes=64)  # 132 bits -> 5 words per token
    ones = np.zeros((1, 5, 1), dtype=np.uint32)  # [Hkv][words][T]
    ones[0, :4, 0] = 0xFFFFFFFF
    ones[0, 4, 0] = 0xF
    assert np.all(oracle.unpack_bits(d, ones, 1) == 63)
    one = np.zeros((1, 5, 1), dtype=np.uint32)
    one[0, 1, 0] = 0x10000000  # bit 60 = index k = 10 = (round 5, group 0), value 1
    got = oracle.unpack_bits(d, one, 1)
    assert got[0, 5, 0, 0] == 1 and got.sum() == 1
    straddle = np.zeros((1, 5, 1), dtype=np.uint32)
    straddle[0, 0, 0] = 1 << 30  # index k = 5 (round 2, group 1) occupies bits 30..35: value 0b110101 = 53
    straddle[0, 1, 0] = 0b1101
    got = oracle.unpack_bits(d, straddle, 1)
    assert got[0, 2, 0, 1] == 53 and got.sum() == 53


def test_unpack_bits_word_planes(oracle_lib):
    """Word w of token t sits at [kv][w][t]: a field set in word 1 of token 2 of KV head 1 belongs to that
    token and head only."""
    d = oracle.dims(1, 4, 2, 11, head_dim=128, n_groups=2, n_codes=64)
    w = np.zeros((2, 5, 3), dtype=np.uint32)
    w[1, 1, 2] = 0x10000000  # bit 60 of token 2's stream: index (round 5, group 0) = 1
    got = oracle.unpack_bits(d, w, 3)
    assert got[1, 5, 2, 0] == 1 and got.sum() == 1


def test_unpack_bits_at_8_bits_one_round_is_the_byte_layout(oracle_lib):
    """With N = 256 and R = 1 a token's bitstream is its 16 code bytes, so the byte layout read as
    little-endian words (and laid out in word planes) unpacks to itself."""
    rng = np.random.default_rng(44)
    d = oracle.dims(1, 4, 3, 1)
    codes = rng.integers(0, 256, size=(3, 1, 11, 16)).astype(np.uint8)
    words = np.ascontiguousarray(codes.reshape(3, 11, 16).view(np.uint32).transpose(0, 2, 1))
    np.testing.assert_array_equal(oracle.unpack_bits(d, words, 11), codes)
    np.testing.assert_array_equal(oracle.unpack(d, codes, 11), codes.astype(np.int32))


def test_pages_setting_attention_matches_torch_sdpa(oracle_lib):
    """The pages' g = 64 / N' = 64 / R = 11 setting end to end: indices drawn here, laid out as bit-packed
    word planes by the workloads generator, unpacked and attended by the oracle, against torch's SDPA over
    keys and values built here by plain indexing."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(45)
    Hkv, R, G, N, W, L = 2, 11, 2, 64, 64, 300
    d = oracle.dims(1, 8, Hkv, R, head_dim=128, n_groups=G, n_codes=N, rope_base=500000.0)
    kcb = rng.standard_normal((Hkv, G, R, N, W)) * 0.5
    vcb = rng.standard_normal((Hkv, G, R, N, W)) * 0.5
    q = rng.standard_normal((1, 8, 128))
    ki = rng.integers(0, N, size=(Hkv, R, L, G)).astype(np.uint8)
    vi = rng.integers(0, N, size=(Hkv, R, L, G)).astype(np.uint8)
    kw, vw = workloads.pack_bits(ki, 6), workloads.pack_bits(vi, 6)
    assert kw.shape == (Hkv, 5, L)  # word planes
    out = oracle.attn_decode(d, q, oracle.unpack_bits(d, kw, L), oracle.unpack_bits(d, vw, L), kcb, vcb,
                             np.zeros(1, np.int64), np.array([L], np.int32), L)
    theta = 500000.0 ** (-np.arange(64) * 2.0 / 128)
    ph = np.exp(1j * np.outer(np.arange(L), theta))
    for kv in range(Hkv):
        K = sum(kcb[kv, np.arange(G)[None, :], r, ki[kv, r]] for r in range(R)).reshape(L, 128)
        V = sum(vcb[kv, np.arange(G)[None, :], r, vi[kv, r]] for r in range(R)).reshape(L, 128)
        Kc = (K[:, 0::2] + 1j * K[:, 1::2]) * ph
        Kr = np.empty_like(K)
        Kr[:, 0::2], Kr[:, 1::2] = Kc.real, Kc.imag
        Q = torch.from_numpy(q[0, 4 * kv:4 * kv + 4])[:, None, :]
        Kt = torch.from_numpy(Kr)[None].expand(4, L, 128).contiguous()
        Vt = torch.from_numpy(V)[None].expand(4, L, 128).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, scale=1 / np.sqrt(128))[:, 0]
        np.testing.assert_allclose(out[0, 4 * kv:4 * kv + 4], ref.numpy(), atol=1e-11)


# ---------------------------------------------------------------------- residual codebook fit (M-step)
def _fit_inputs(rng, Hkv, R, n, G=2, D=16, N=16):
    d = oracle.dims(1, 4, Hkv, R, head_dim=D, n_groups=G, n_codes=N)
    W = D // G
    x = rng.standard_normal((Hkv, n, D))
    return d, x, W


def test_codebook_update_r1_is_one_lloyd_iteration(oracle_lib):
    """R = 1: encode + update is one Lloyd k-means iteration, checked against scikit-learn's KMeans."""
    sk = pytest.importorskip("sklearn.cluster")
    rng = np.random.default_rng(30)
    Hkv, n, G, D, N = 2, 400, 2, 16, 16
    d, x, W = _fit_inputs(rng, Hkv, 1, n, G, D, N)
    # initial codewords are data points, so every cluster keeps at least one member
    pick = rng.choice(n, size=N, replace=False)
    cb = np.stack([np.stack([x[kv, pick, g * W:(g + 1) * W] for g in range(G)]) for kv in range(Hkv)])[:, :, None]
    codes = oracle.encode_greedy(d, x, cb)
    new = oracle.codebook_update(d, x, cb, codes)
    import warnings
    for kv in range(Hkv):
        for g in range(G):
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                km = sk.KMeans(n_clusters=N, init=cb[kv, g, 0], n_init=1, max_iter=1, tol=0.0,
                               algorithm="lloyd").fit(x[kv, :, g * W:(g + 1) * W])
            np.testing.assert_allclose(new[kv, g, 0], km.cluster_centers_, rtol=1e-10, atol=1e-12)


def test_codebook_update_is_the_round_least_squares_solution(oracle_lib):
    """Each updated codeword minimizes its round's squared error for the given assignment (residuals
    built by decoding the earlier rounds); unused codewords keep their value; counts are the histogram."""
    rng = np.random.default_rng(31)
    Hkv, R, n, G, D, N = 1, 2, 60, 2, 16, 16
    d, x, W = _fit_inputs(rng, Hkv, R, n, G, D, N)
    cb = rng.standard_normal((Hkv, G, R, N, W)) * 0.5
    codes = rng.integers(0, N - 2, size=(Hkv, R, n, G)).astype(np.uint8)  # codes N-2, N-1 never used
    new, counts = oracle.codebook_update(d, x, cb, codes, want_counts=True)
    for r in range(R):
        cb_before = cb.copy()
        cb_before[:, :, r:] = 0.0  # decode of rounds < r only
        res = x - oracle.decode(d, cb_before, codes, n)  # round-r residual of every token
        for g in range(G):
            np.testing.assert_array_equal(counts[0, g, r], np.bincount(codes[0, r, :, g], minlength=N))
            for l in range(N):
                members = res[0, codes[0, r, :, g] == l, g * W:(g + 1) * W]
                if len(members) == 0:
                    np.testing.assert_array_equal(new[0, g, r, l], cb[0, g, r, l])
                    continue
                f = lambda c: float(((members - c[None, :]) ** 2).sum())
                f0 = f(new[0, g, r, l])
                for _ in range(4):
                    delta = rng.standard_normal(W) * 1e-3
                    assert f(new[0, g, r, l] + delta) > f0
                assert f0 <= f(cb[0, g, r, l]) + 1e-12


def test_codebook_update_fixed_point_on_exact_codewords(oracle_lib):
    rng = np.random.default_rng(32)
    Hkv, n, G, D, N = 2, 200, 2, 16, 16
    d = oracle.dims(1, 4, Hkv, 1, head_dim=D, n_groups=G, n_codes=N)
    cb = rng.standard_normal((Hkv, G, 1, N, D // G))
    codes = np.tile(np.arange(n) % N, (Hkv, 1, G, 1)).transpose(0, 1, 3, 2).astype(np.uint8)  # every code used
    x = oracle.decode(d, cb, codes, n)
    got = oracle.encode_greedy(d, x, cb)
    np.testing.assert_array_equal(got, codes)
    np.testing.assert_allclose(oracle.codebook_update(d, x, cb, got), cb, rtol=0, atol=1e-14)


def test_em_iterations_do_not_increase_r1_error(oracle_lib):
    """Lloyd's iteration never increases the squared error (R = 1)."""
    rng = np.random.default_rng(33)
    Hkv, n, G, D, N = 1, 500, 2, 16, 16
    d, x, W = _fit_inputs(rng, Hkv, 1, n, G, D, N)
    cb = rng.standard_normal((Hkv, G, 1, N, W))
    errs = []
    for _ in range(6):
        codes = oracle.encode_greedy(d, x, cb)
        errs.append(float(((x - oracle.decode(d, cb, codes, n)) ** 2).sum()))
        cb = oracle.codebook_update(d, x, cb, codes)
    assert all(b <= a + 1e-9 for a, b in zip(errs, errs[1:]))
    assert errs[-1] < errs[0]


# ------------------------------------------------------------------------------------ page figures
def test_page_figures_bit_rate_and_memory():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)
    # bits per scalar of an index shared by g dims with N' codes and R rounds: R * log2(N') / g
    for row in fig["bit_rate"]:
        assert row["R"] * math.log2(row["n_codes"]) / row["g"] == pytest.approx(row["avg_bit"], abs=row["tol"])
    # this layout: 8-dim groups, N = 256 -> R bits per scalar; 2-bit keeps 2/16 of an fp16 cache
    for R in (1, 2):
        cfg = workloads.custom("fig", 1, 32, 8, (1000,), R, "float16", 0)
        fp16_bytes = 2 * 8 * 1000 * 128 * 2
        assert workloads.code_bytes(cfg, 1000) * 8 / (2 * 8 * 1000 * 128) == R
        if R == 2:
            assert 1 - workloads.code_bytes(cfg, 1000) / fp16_bytes == pytest.approx(fig["fp16_cut_2bit"])
