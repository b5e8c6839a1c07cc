"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: per (b, q head) output row, max_i |gpu - oracle| / max_i |oracle| <= 2e-3 for fp16 storage
and 1e-5 for fp32 storage; the unpack is compared bit-exactly. Inputs come from workloads.make_inputs,
shared by both sides; the oracle sees the same fp16/fp32 values converted exactly to fp64.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"float16": 2e-3, "float32": 1e-5}
THREADS = 16


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vector_quantized_kv_amd as m
    m.lib()
    return m


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def rowwise_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    num = np.abs(got - ref).reshape(-1, ref.shape[-1]).max(-1)
    den = np.abs(ref).reshape(-1, ref.shape[-1]).max(-1)
    den = np.where(den == 0, 1.0, den)
    return (num / den).max()


def run_attn(vq, cfg, inp):
    d = vq.dims_of(cfg)
    layer = vq.Layer(d, inp)
    out = layer.attn_decode()
    torch.cuda.synchronize()
    return out.cpu().numpy()


CONFIG_NAMES = list(workloads.CONFIGS)


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_attn_decode_matches_oracle_full_configs(vq, name):
    cfg = workloads.CONFIGS[name]
    announce(f"attn_decode {name}")
    inp = workloads.make_inputs(cfg)
    got = run_attn(vq, cfg, inp)
    ref = oracle.run_config(cfg, inp, n_threads=THREADS)
    err = rowwise_rel_err(got, ref)
    print(f"{name}: max row-relative error {err:.3e} (tol {TOL[cfg.dtype]})", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= TOL[cfg.dtype]


EDGE = [
    ("one_token_f32", 1, (1,), 2, "float32"),
    ("ragged_tails_f32", 3, (1023, 1024, 1025), 1, "float32"),
    ("ragged_small_f16", 4, (1, 64, 65, 3000), 2, "float16"),
    ("empty_sequence_f16", 3, (700, 0, 2049), 2, "float16"),
    ("split_boundary_r1_f16", 2, (2048, 4096), 1, "float16"),
    # more than 32 splits per (sequence, KV head): the last workgroup's merge runs several chunks and
    # rescales the earlier ones by the running maximum
    ("long_merge_chunks_f16", 1, (300000,), 2, "float16"),
    ("long_merge_chunks_r1_f16", 2, (700001, 5000), 1, "float16"),
    ("long_merge_chunks_f32", 1, (150000,), 2, "float32"),
]


@pytest.mark.parametrize("name,B,lengths,R,dtype", EDGE)
def test_attn_decode_edge_cases(vq, name, B, lengths, R, dtype):
    announce(f"attn_decode edge {name} lengths={lengths} R={R} {dtype}")
    cfg = workloads.custom(name, B, 8, 2, lengths, R, dtype, 100 + len(name))
    inp = workloads.make_inputs(cfg)
    got = run_attn(vq, cfg, inp)
    ref = oracle.run_config(cfg, inp, n_threads=THREADS)
    for b, L in enumerate(lengths):
        if L == 0:
            assert np.all(got[b] == 0.0)
    err = rowwise_rel_err(got, ref)
    print(f"{name}: {err:.3e}", flush=True)
    assert err <= TOL[dtype]


# 8 KV heads, as in the benchmark: 64K and 96K tokens give every wave 4 and 6 key blocks (key sweeps of two blocks
# with the later sweeps skipped); the ragged batch mixes even and odd block counts within one workgroup.
SWEEP_CASES = [("sweeps_4_blocks_r2", 1, (65536,), 2), ("sweeps_6_blocks_r2", 1, (98304,), 2),
               ("sweeps_6_blocks_r1", 1, (98304,), 1), ("sweeps_mixed_r2", 3, (50000, 30000, 12000), 2)]


@pytest.mark.parametrize("name,B,lengths,R", SWEEP_CASES)
def test_attn_decode_block_counts(vq, name, B, lengths, R):
    announce(f"attn_decode {name} lengths={lengths} R={R}")
    cfg = workloads.custom(name, B, 32, 8, lengths, R, "float16", 200 + len(name))
    inp = workloads.make_inputs(cfg)
    got = run_attn(vq, cfg, inp)
    ref = oracle.run_config(cfg, inp, n_threads=THREADS)
    err = rowwise_rel_err(got, ref)
    print(f"{name}: {err:.3e}", flush=True)
    assert err <= TOL["float16"]


@pytest.mark.parametrize("name", ["tiny_1k_r2_f32", "llama8b_8k_r2", "llama8b_32k_r1", "ragged16_r2"])
def test_unpack_bit_exact(vq, name):
    cfg = workloads.CONFIGS[name]
    announce(f"debug_unpack {name}")
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    for key in ("k_codes", "v_codes"):
        codes = torch.from_numpy(inp[key]).cuda()
        got = vq.debug_unpack(d, codes, int(inp["total_tokens"]))
        torch.cuda.synchronize()
        ref = oracle.unpack(oracle.dims_of(cfg), inp[key], int(inp["total_tokens"]))
        np.testing.assert_array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("dtype,R,tol", [("float32", 2, 1e-6), ("float16", 1, 1e-3), ("float16", 2, 1e-3)])
def test_qcodebook_table_matches_oracle(vq, dtype, R, tol):
    announce(f"qcodebook_table {dtype} R={R}")
    cfg = workloads.custom("tab", 2, 8, 2, (5, 5), R, dtype, 21)
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    dt = torch.float16 if dtype == "float16" else torch.float32
    q = torch.from_numpy(inp["q"]).cuda().to(dt)
    kcb = torch.from_numpy(inp["k_cb"]).cuda().to(dt)
    got = vq.qcodebook_table(d, q, kcb)
    torch.cuda.synchronize()
    ref = oracle.table(oracle.dims_of(cfg), inp["q"], inp["k_cb"])
    g = got.float().cpu().numpy().astype(np.float64)
    for b in range(2):
        for h in range(8):
            err = np.abs(g[b, h] - ref[b, h]).max() / np.abs(ref[b, h]).max()
            assert err <= tol, (b, h, err)


@pytest.mark.parametrize("dtype,R,signed", [("float32", 2, False), ("float32", 1, True), ("float16", 2, False),
                                            ("float16", 1, True), ("float16", 1, False), ("float16", 2, True),
                                            ("float16", 2, "mixed")])
def test_value_reduce_matches_oracle(vq, dtype, R, signed):
    """Weights of either sign; "mixed": negative only in a few tokens past token 2048 of the first sequence (its
    second 2048-token work item in fp32 storage, its only 4096-token item in fp16 storage), so that one workgroup
    takes the signed bins and the others the non-negative ones."""
    announce(f"value_reduce {dtype} R={R} signed={signed}")
    cfg = workloads.custom("vr", 3, 8, 2, (2500, 1, 1024), R, dtype, 22)
    inp = workloads.make_inputs(cfg)
    L = int(inp["max_len"])
    rng = np.random.default_rng(23)
    p = rng.uniform(-1 if signed is True else 0, 1, size=(3, 8, L)).astype(np.float32)
    if signed == "mixed":
        p[0, 3, 2100:2110] *= -1.0
    d = vq.dims_of(cfg)
    dt = torch.float16 if dtype == "float16" else torch.float32
    got = vq.value_reduce(d, torch.from_numpy(p).cuda(), torch.from_numpy(inp["v_codes"]).cuda(),
                          torch.from_numpy(inp["v_cb"]).cuda().to(dt), torch.from_numpy(inp["seq_start"]).cuda(),
                          torch.from_numpy(inp["seq_len"]).cuda(), L, int(inp["total_tokens"]))
    torch.cuda.synchronize()
    ref = oracle.value_reduce(oracle.dims_of(cfg), p, inp["v_codes"], inp["v_cb"], inp["seq_start"], inp["seq_len"], L)
    err = rowwise_rel_err(got.cpu().numpy(), ref)
    print(f"value_reduce {dtype} R={R}: {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,R,signed", [("float16", 2, False), ("float16", 1, True), ("float32", 2, True)])
def test_value_reduce_work_item_edges(vq, dtype, R, signed):
    """Sequence lengths at and around the work-item sizes (4096 tokens in fp16 storage, 2048 in fp32): exactly one
    and two items, one token past an item, one token short of one, and three items plus one token."""
    announce(f"value_reduce item edges {dtype} R={R} signed={signed}")
    cfg = workloads.custom("vr_edges", 5, 8, 2, (8192, 4097, 4095, 4096, 12289), R, dtype, 26)
    inp = workloads.make_inputs(cfg)
    L = int(inp["max_len"])
    rng = np.random.default_rng(27)
    p = rng.uniform(-1 if signed else 0, 1, size=(5, 8, L)).astype(np.float32)
    d = vq.dims_of(cfg)
    dt = torch.float16 if dtype == "float16" else torch.float32
    got = vq.value_reduce(d, torch.from_numpy(p).cuda(), torch.from_numpy(inp["v_codes"]).cuda(),
                          torch.from_numpy(inp["v_cb"]).cuda().to(dt), torch.from_numpy(inp["seq_start"]).cuda(),
                          torch.from_numpy(inp["seq_len"]).cuda(), L, int(inp["total_tokens"]))
    torch.cuda.synchronize()
    ref = oracle.value_reduce(oracle.dims_of(cfg), p, inp["v_codes"], inp["v_cb"], inp["seq_start"], inp["seq_len"], L)
    err = rowwise_rel_err(got.cpu().numpy(), ref)
    print(f"value_reduce item edges {dtype} R={R}: {err:.3e}", flush=True)
    assert err <= TOL[dtype]


SOFTMAX_P = [("float32", 2, 3.0), ("float32", 1, 3.0), ("float32", 2, 6.0), ("float16", 2, 3.0)]


@pytest.mark.parametrize("dtype,R,score_std", SOFTMAX_P)
def test_value_reduce_softmax_weights(vq, dtype, R, score_std):
    """Softmax-shaped weights (scores of standard deviation 3 or 6 over each sequence): a few weights near the
    split maximum and many orders of magnitude below it, the case where the fixed-point bins round most."""
    announce(f"value_reduce softmax p {dtype} R={R} std={score_std}")
    cfg = workloads.custom("vr_sm", 3, 8, 2, (5000, 700, 3072), R, dtype, 24 + R)
    inp = workloads.make_inputs(cfg)
    L = int(inp["max_len"])
    rng = np.random.default_rng(25 + R)
    s = rng.normal(0.0, score_std, size=(3, 8, L))
    p = np.zeros((3, 8, L), dtype=np.float32)
    for b, n in enumerate(int(x) for x in inp["seq_len"]):
        e = np.exp(s[b, :, :n] - s[b, :, :n].max(-1, keepdims=True))
        p[b, :, :n] = (e / e.sum(-1, keepdims=True)).astype(np.float32)
    d = vq.dims_of(cfg)
    dt = torch.float16 if dtype == "float16" else torch.float32
    got = vq.value_reduce(d, torch.from_numpy(p).cuda(), torch.from_numpy(inp["v_codes"]).cuda(),
                          torch.from_numpy(inp["v_cb"]).cuda().to(dt), torch.from_numpy(inp["seq_start"]).cuda(),
                          torch.from_numpy(inp["seq_len"]).cuda(), L, int(inp["total_tokens"]))
    torch.cuda.synchronize()
    ref = oracle.value_reduce(oracle.dims_of(cfg), p, inp["v_codes"], inp["v_cb"], inp["seq_start"], inp["seq_len"], L)
    err = rowwise_rel_err(got.cpu().numpy(), ref)
    print(f"value_reduce softmax p {dtype} R={R} std={score_std}: {err:.3e}", flush=True)
    assert err <= TOL[dtype]


def test_rope_table_matches_fp64(vq):
    announce("rope_table")
    d = vq.make_dims(1, 4, 1, 1)
    n = 131072 + 5
    raw = vq.rope_table(d, n).cpu().numpy()
    theta = 500000.0 ** (-np.arange(64) * 2.0 / 128)
    fine = np.exp(1j * np.outer(np.arange(64), theta))          # [f][j]
    coarse = np.exp(1j * np.outer(64.0 * np.arange((n + 63) // 64), theta))
    fine32 = raw[:8192].view(np.complex64).reshape(64, 64)       # pair-major [j][f]
    f32g = raw[8192:16384].view(np.complex64).reshape(16, 2, 64, 2)  # [g][h][f][p], pair 4g + 2h + p
    fine32g = f32g.transpose(2, 0, 1, 3).reshape(64, 64)             # [f][j]
    coarse32 = raw[16384:].view(np.complex64).reshape(-1, 64)
    assert coarse32.shape[0] == coarse.shape[0]
    # every entry rounded once from the fp64 phase: within half an fp32 ulp of values of magnitude <= 1
    assert np.abs(fine32 - fine.T).max() < 1e-7
    assert np.abs(fine32g - fine).max() < 1e-7
    assert np.abs(coarse32 - coarse).max() < 1e-7


def test_workspace_too_small_is_rejected(vq):
    announce("workspace too small")
    cfg = workloads.custom("ws", 1, 8, 2, (3000,), 1, "float16", 24)
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    layer = vq.Layer(d, inp)
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(vq.CommVQError) as ei:
        vq.attn_decode(d, layer.q, layer.k_codes, layer.v_codes, layer.k_cb, layer.v_cb, layer.seq_start,
                       layer.seq_len, layer.max_len, layer.total_tokens, layer.rope, layer.rope_positions, small)
    assert ei.value.status == vq.EWORKSPACE


def test_repeat_calls_are_consistent(vq):
    announce("repeat calls")
    cfg = workloads.CONFIGS["llama8b_8k_r2"]
    inp = workloads.make_inputs(cfg)
    layer = vq.Layer(vq.dims_of(cfg), inp)
    a = layer.attn_decode().clone()
    b = layer.attn_decode().clone()
    torch.cuda.synchronize()
    assert rowwise_rel_err(b.cpu().numpy(), a.cpu().numpy().astype(np.float64)) <= 1e-5


def encode_inputs(Hkv, n, R, dtype, seed):
    rng = np.random.default_rng(seed)
    cb = (rng.standard_normal((Hkv, 16, R, 256, 8), dtype=np.float32) * np.float32(0.5)).astype(dtype)
    x = (rng.standard_normal((Hkv, n, 128), dtype=np.float32) * np.float32(0.7)).astype(dtype)
    return x, cb


@pytest.mark.parametrize("dtype,R,n", [("float32", 2, 300), ("float16", 1, 513), ("float16", 2, 1000)])
def test_encode_greedy_choices_are_optimal(vq, dtype, R, n):
    announce(f"encode_greedy {dtype} R={R} n={n}")
    Hkv = 2
    x, cb = encode_inputs(Hkv, n, R, dtype, 30 + R)
    d = vq.make_dims(1, 4 * Hkv, Hkv, R, dtype)
    got = vq.encode_greedy(d, torch.from_numpy(x).cuda(), torch.from_numpy(cb).cuda())
    torch.cuda.synchronize()
    codes = got.cpu().numpy()
    od = oracle.dims(1, 4 * Hkv, Hkv, R)
    chosen, best, second = oracle.encode_eval(od, x, cb, codes)
    # the GPU decides in fp32, the oracle replays in fp64: every choice is a minimum up to fp32 rounding,
    # and where the fp64 minimum is unique by a clear margin the GPU picked exactly it
    scale = best + 1e-3
    assert np.all(chosen - best <= 1e-5 * scale)
    unique = (second - best) > 1e-4 * scale
    assert unique.mean() > 0.95
    np.testing.assert_array_equal(chosen[unique], best[unique])
    ref = oracle.encode_greedy(od, x, cb)
    first_round_unique = unique[:, 0]
    np.testing.assert_array_equal(codes[:, 0][first_round_unique], ref[:, 0][first_round_unique])


def test_encode_greedy_recovers_exact_codewords_and_appends_in_place(vq):
    announce("encode_greedy exact recovery + append")
    Hkv, n, R = 2, 200, 1
    rng = np.random.default_rng(40)
    cb = (rng.standard_normal((Hkv, 16, R, 256, 8), dtype=np.float32) * np.float32(0.5)).astype(np.float16)
    idx = rng.integers(0, 256, size=(Hkv, R, n, 16)).astype(np.uint8)
    od = oracle.dims(1, 4 * Hkv, Hkv, R)
    x = oracle.decode(od, cb, idx, n).astype(np.float16)  # exact: one fp16 codeword per group
    d = vq.make_dims(1, 4 * Hkv, Hkv, R, "float16")
    big = torch.full((Hkv, R, n + 9, 16), 0xAB, dtype=torch.uint8, device="cuda")
    vq.encode_greedy(d, torch.from_numpy(x).cuda(), torch.from_numpy(cb).cuda(), codes=big, first_row=5)
    torch.cuda.synchronize()
    out = big.cpu().numpy()
    np.testing.assert_array_equal(out[:, :, 5:5 + n], idx)
    assert np.all(out[:, :, :5] == 0xAB) and np.all(out[:, :, 5 + n:] == 0xAB)


@pytest.mark.parametrize("dtype,R,n", [("float32", 2, 3000), ("float16", 1, 2500), ("float16", 2, 4001)])
def test_codebook_update_matches_oracle(vq, dtype, R, n):
    """The M-step on the GPU against the oracle's for the same assignment (codes 250..255 unused)."""
    announce(f"codebook_update {dtype} R={R} n={n}")
    Hkv = 2
    x, cb = encode_inputs(Hkv, n, R, dtype, 50 + R)
    rng = np.random.default_rng(60 + R)
    codes = rng.integers(0, 250, size=(Hkv, R, n, 16)).astype(np.uint8)
    d = vq.make_dims(1, 4 * Hkv, Hkv, R, dtype)
    args = (torch.from_numpy(x).cuda(), torch.from_numpy(codes).cuda(), torch.from_numpy(cb).cuda())
    got = vq.codebook_update(d, *args)
    again = vq.codebook_update(d, *args)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    np.testing.assert_array_equal(again.cpu().numpy(), got)  # exact sums: no dependence on the order of adds
    od = oracle.dims(1, 4 * Hkv, Hkv, R)
    ref, counts = oracle.codebook_update(od, x, cb, codes, want_counts=True)
    used = counts > 0
    assert not used[..., 250:].any() and used[..., :250].all()
    np.testing.assert_array_equal(got[..., 250:, :], cb[..., 250:, :])  # unused codewords are kept
    if dtype == "float32":
        np.testing.assert_allclose(got.astype(np.float64), ref, rtol=1e-5, atol=1e-6)
    else:
        # fp32 sums rounded once to fp16: within one fp16 ulp of the fp64 mean
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)


def test_fit_codebook_r1_error_never_increases(vq):
    """E-step (encode_greedy) + M-step (codebook_update) on the GPU is Lloyd's iteration at R = 1: the squared
    error, measured by the oracle's decode, never increases."""
    announce("fit_codebook R=1")
    Hkv, n, R = 1, 4000, 1
    x, cb = encode_inputs(Hkv, n, R, "float32", 70)
    d = vq.make_dims(1, 4, Hkv, R, "float32")
    od = oracle.dims(1, 4, Hkv, R)
    xt, cur = torch.from_numpy(x).cuda(), torch.from_numpy(cb).cuda()
    errs = []
    for _ in range(5):
        cur_np = cur.cpu().numpy()
        cur, codes = vq.fit_codebook(d, xt, cur, 1)
        torch.cuda.synchronize()
        errs.append(float(((x - oracle.decode(od, cur_np, codes.cpu().numpy(), n)) ** 2).sum()))
    print("fit errors", errs, flush=True)
    assert all(b <= a * (1 + 1e-6) for a, b in zip(errs, errs[1:]))
    assert errs[-1] < 0.9 * errs[0]


def split_tokens(B, L, n_kv):
    """The library's split sizing: 512 tokens per block of 8 waves x 64, 1..8 blocks per wave, ~one item per CU."""
    blocks = max(1, min(8, -(-(L * B * n_kv) // (256 * 512))))
    return 512 * blocks


@pytest.mark.parametrize("R", [1, 2])
def test_split_size_does_not_change_the_result(vq, R):
    # one sequence alone (512-token splits) and as 8 copies in one batch (2048-token splits)
    announce(f"split-size independence R={R}")
    L, B = 8192, 8
    cfg1 = workloads.custom("split_b1", 1, 32, 8, (L,), R, "float16", 77 + R)
    inp1 = workloads.make_inputs(cfg1)
    cfg8 = workloads.custom("split_b8", B, 32, 8, (L,) * B, R, "float16", 77 + R)
    inp8 = dict(inp1, q=np.repeat(inp1["q"], B, axis=0), seq_start=np.zeros(B, np.int64),
                seq_len=np.full(B, L, np.int32))
    assert split_tokens(1, L, 8) != split_tokens(B, L, 8)
    out1 = run_attn(vq, cfg1, inp1)
    out8 = run_attn(vq, cfg8, inp8)
    for b in range(B):
        np.testing.assert_array_equal(out8[b], out8[0])  # same inputs, same split: same bits
    err = rowwise_rel_err(out8[0], out1[0].astype(np.float64))
    print(f"split 512 vs 2048 tokens: max row-relative difference {err:.3e}", flush=True)
    assert err <= TOL["float16"]
    ref = oracle.run_config(cfg1, inp1, n_threads=THREADS)
    assert rowwise_rel_err(out1, ref) <= TOL["float16"]


def counting_value_codebook(Hkv, G, R, N, W, dtype):
    """Codeword l of residual r holds l in dim r of its group and zeros elsewhere: a decode reveals the indices."""
    cb = np.zeros((Hkv, G, R, N, W), dtype=dtype)
    for r in range(R):
        cb[:, :, r, :, r] = np.arange(N, dtype=np.float32).astype(dtype)
    return cb


def read_indices_back(vq, cfg, unpack):
    """64 one-token sequences at scattered rows: p = 1, so out = the decoded value, i.e. the stored indices."""
    B = 64
    inp = workloads.make_inputs(cfg)
    T = int(inp["total_tokens"])
    rows = (np.arange(B, dtype=np.int64) * 37 + 5) % T
    G, R, N, W = cfg.n_groups, cfg.n_residuals, cfg.n_codes, cfg.group_dim
    inp = dict(inp, v_cb=counting_value_codebook(cfg.n_kv_heads, G, R, N, W, np.dtype(cfg.dtype)),
               q=np.repeat(inp["q"][:1], B, axis=0), seq_start=rows, seq_len=np.ones(B, np.int32),
               max_len=np.int32(1))
    cfgB = workloads.custom(cfg.name + "_b64", B, cfg.n_q_heads, cfg.n_kv_heads, (1,) * B, R, cfg.dtype, cfg.seed,
                            n_groups=G, n_codes=N)
    got = run_attn(vq, cfgB, inp)  # [B][Hq][D]
    idx = unpack(inp["v_codes"], T)  # [Hkv][R][T][G]
    for h in range(cfg.n_q_heads):
        kv = h // 4
        for r in range(R):
            want = idx[kv, r][rows]  # [B][G]
            np.testing.assert_array_equal(got[:, h, np.arange(G) * W + r], want.astype(np.float32))


@pytest.mark.parametrize("dtype,R", [("float16", 1), ("float16", 2), ("float32", 2)])
def test_attention_reads_every_value_index_back(vq, dtype, R):
    announce(f"value indices through attention {dtype} R={R}")
    cfg = workloads.custom("counting", 1, 8, 2, (3000,), R, dtype, 31 + R)
    d = oracle.dims_of(cfg)
    read_indices_back(vq, cfg, lambda codes, T: oracle.unpack(d, codes, T))


@pytest.mark.parametrize("R", [1, 2])
def test_attn_decode_sixteen_kv_heads(vq, R):
    # 16 KV heads (64 q heads) in a batch of 3: two heads per XCD in the grid's dealing order
    announce(f"attn_decode 16 KV heads R={R}")
    cfg = workloads.custom("kv16", 3, 64, 16, (5000, 1, 2049), R, "float16", 90 + R)
    inp = workloads.make_inputs(cfg)
    got = run_attn(vq, cfg, inp)
    err = rowwise_rel_err(got, oracle.run_config(cfg, inp, n_threads=THREADS))
    print(f"kv16 R={R}: {err:.3e}", flush=True)
    assert err <= TOL["float16"]
