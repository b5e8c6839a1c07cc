"""GPU parity of the bit-packed layout (one index per 64 dims, N = 64 codewords, R residual rounds: the
CommVQ pages' own code shape) against the fp64 oracle, through the C ABI.

Same bars as the byte layout: per (b, q head) output row, max_i |gpu - oracle| / max_i |oracle| <= 2e-3
(fp16 codebooks), and the unpack of the bit-packed records compared bit-exactly with the oracle's.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3
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


def pages_cfg(name, B, lengths, R, seed, n_kv=2):
    return workloads.custom(name, B, 4 * n_kv, n_kv, lengths, R, "float16", seed, n_groups=2, n_codes=64)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 21, 32])
def test_pages_unpack_bit_exact(vq, R):
    cfg = pages_cfg(f"unpack_r{R}", 2, (777, 1), R, 300 + R)
    announce(f"debug_unpack bit-packed R={R}")
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    T = int(inp["total_tokens"])
    for key in ("k_codes", "v_codes"):
        words = torch.from_numpy(inp[key].view(np.int32)).cuda()
        got = vq.debug_unpack(d, words, T)
        torch.cuda.synchronize()
        ref = oracle.unpack_bits(oracle.dims_of(cfg), inp[key], T)
        np.testing.assert_array_equal(got.cpu().numpy(), ref.astype(np.int32))


def check_attn(vq, cfg, inp, repeat=1):
    layer = vq.Layer(vq.dims_of(cfg), inp)
    outs = []
    for _ in range(repeat):
        outs.append(layer.attn_decode().clone())
    torch.cuda.synchronize()
    got = outs[0].cpu().numpy()
    for o in outs[1:]:  # the arrival counters reset: a repeated call gives the same bits
        np.testing.assert_array_equal(o.cpu().numpy(), got)
    ref = oracle.run_config(cfg, inp, n_threads=THREADS)
    assert np.all(np.isfinite(got))
    for b, L in enumerate(inp["seq_len"]):
        if L == 0:
            assert np.all(got[b] == 0.0)
    err = rowwise_rel_err(got, ref)
    print(f"{cfg.name}: max row-relative error {err:.3e} (tol {TOL})", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("name", list(workloads.PAGES_CONFIGS))
def test_pages_attn_matches_oracle_configs(vq, name):
    cfg = workloads.PAGES_CONFIGS[name]
    announce(f"attn_decode bit-packed {name}")
    check_attn(vq, cfg, workloads.make_inputs(cfg), repeat=2)


PAGES_EDGE = [
    # name, B, lengths, R. The kernel is instantiated per last-window size T = R - 8 (ceil(R / 8) - 1): T <= 4 takes
    # one pass over both groups, T > 4 two one-group passes; every T from 1 to 8 appears below.
    ("pages_r1_ragged", 4, (1, 64, 65, 3000), 1),        # T = 1: a single pass over both groups
    ("pages_r2_tail", 2, (1500, 64), 2),                 # T = 2
    ("pages_r4_whole_pass", 2, (513, 4096), 4),          # T = 4: the largest both-group pass
    ("pages_r5_empty_seq", 3, (700, 0, 2049), 5),        # T = 5: the smallest one-group tail; an empty sequence
    ("pages_r14_tail6", 2, (3000, 777), 14),             # a full window, then T = 6
    ("pages_r15_tail7", 1, (2500,), 15),                 # a full window, then T = 7
    ("pages_r8_one_window", 2, (129, 2048), 8),          # T = 8: one full window, no tail pass
    ("pages_r13_ragged", 2, (4097, 123), 13),
    ("pages_r11_split_boundary", 2, (2048, 4096), 11),
    ("pages_r32_max", 1, (5000,), 32),                   # the largest R: twelve-word records, four full windows
    ("pages_r21_long_merge", 1, (300000,), 21),          # more than 32 splits per (sequence, KV head)
]


@pytest.mark.parametrize("name,B,lengths,R", PAGES_EDGE)
def test_pages_attn_edge_cases(vq, name, B, lengths, R):
    announce(f"attn_decode bit-packed edge {name} lengths={lengths} R={R}")
    cfg = pages_cfg(name, B, lengths, R, 400 + len(name) + R)
    check_attn(vq, cfg, workloads.make_inputs(cfg))


def test_pages_attn_ragged_batch(vq):
    # 16 sequences of 4096 .. 65536 tokens at the Llama-3.1-8B layer shape (the byte layout's ragged16_r2)
    announce("attn_decode bit-packed ragged batch of 16, R=11")
    cfg = workloads.Config("pages_ragged16_r11", 16, 32, 8, None, 11, "float16", 25, n_groups=2, n_codes=64,
                           ragged_range=(4096, 65536))
    check_attn(vq, cfg, workloads.make_inputs(cfg))


@pytest.mark.parametrize("n_kv,B,lengths,R", [(1, 1, (2500,), 11), (3, 2, (1500, 777), 21)])
def test_pages_attn_kv_head_counts(vq, n_kv, B, lengths, R):
    # one KV head (4 q heads), and an odd count that does not divide the 8 XCDs the grid is dealt to
    announce(f"attn_decode bit-packed n_kv={n_kv} lengths={lengths} R={R}")
    cfg = pages_cfg(f"pages_kv{n_kv}", B, lengths, R, 500 + n_kv, n_kv=n_kv)
    check_attn(vq, cfg, workloads.make_inputs(cfg))


def test_pages_split_size_does_not_change_the_result(vq):
    # one sequence alone (512-token splits) and as 8 copies in one batch (2048-token splits)
    announce("bit-packed split-size independence")
    L, B = 8192, 8
    cfg1 = pages_cfg("pages_split_b1", 1, (L,), 11, 91, n_kv=8)
    inp1 = workloads.make_inputs(cfg1)
    cfg8 = pages_cfg("pages_split_b8", B, (L,) * B, 11, 91, n_kv=8)
    inp8 = dict(inp1, q=np.repeat(inp1["q"], B, axis=0), seq_start=np.zeros(B, np.int64),
                seq_len=np.full(B, L, np.int32))
    out = []
    for cfg, inp in ((cfg1, inp1), (cfg8, inp8)):
        layer = vq.Layer(vq.dims_of(cfg), inp)
        out.append(layer.attn_decode().cpu().numpy())
    for b in range(B):
        np.testing.assert_array_equal(out[1][b], out[1][0])
    err = rowwise_rel_err(out[1][0], out[0][0].astype(np.float64))
    print(f"bit-packed split 512 vs 2048 tokens: max row-relative difference {err:.3e}", flush=True)
    assert err <= TOL
    assert rowwise_rel_err(out[0], oracle.run_config(cfg1, inp1, n_threads=THREADS)) <= TOL


@pytest.mark.parametrize("R", [5, 21])
def test_pages_attention_reads_every_value_index_back(vq, R):
    # 64 one-token sequences: p = 1, and codeword l of residual r holds l in dim r of its group, so each output
    # row is the token's stored value indices (read through the window unpack, the gathers and the value MFMAs)
    from test_gpu_parity import read_indices_back
    announce(f"bit-packed value indices through attention R={R}")
    cfg = pages_cfg("pages_counting", 1, (3000,), R, 61 + R)
    d = oracle.dims_of(cfg)
    read_indices_back(vq, cfg, lambda words, T: oracle.unpack_bits(d, words, T))


def pages_encode_inputs(Hkv, n, R, seed):
    rng = np.random.default_rng(seed)
    cb = (rng.standard_normal((Hkv, 2, R, 64, 64), dtype=np.float32) * np.float32(0.5)).astype(np.float16)
    x = (rng.standard_normal((Hkv, n, 128), dtype=np.float32) * np.float32(0.7)).astype(np.float16)
    return x, cb


@pytest.mark.parametrize("R,n", [(1, 300), (11, 1000), (21, 513)])
def test_pages_encode_greedy_choices_are_optimal(vq, R, n):
    # the greedy encoder writing bit-packed records: read back through the oracle's unpack, every choice is a
    # minimum of the fp64 replay up to fp32 rounding, and clear minima are picked exactly
    announce(f"encode_greedy bit-packed R={R} n={n}")
    Hkv = 2
    x, cb = pages_encode_inputs(Hkv, n, R, 70 + R)
    d = vq.make_dims(1, 4 * Hkv, Hkv, R, "float16", n_groups=2, n_codes=64)
    words = vq.encode_greedy(d, torch.from_numpy(x).cuda(), torch.from_numpy(cb).cuda())
    torch.cuda.synchronize()
    od = oracle.dims(1, 4 * Hkv, Hkv, R, n_groups=2, n_codes=64)
    codes = oracle.unpack_bits(od, words.cpu().numpy().view(np.uint32), n)
    chosen, best, second = oracle.encode_eval(od, x, cb, codes)
    scale = best + 1e-3
    assert np.all(chosen - best <= 1e-5 * scale)
    unique = (second - best) > 1e-4 * scale
    assert unique.mean() > 0.95
    np.testing.assert_array_equal(chosen[unique], best[unique])
    ref = oracle.encode_greedy(od, x, cb)
    first_round_unique = unique[:, 0]
    np.testing.assert_array_equal(codes[:, 0][first_round_unique], ref[:, 0][first_round_unique])


def test_pages_encode_greedy_recovers_codewords_and_appends_in_place(vq):
    announce("encode_greedy bit-packed exact recovery + append")
    Hkv, n, R = 2, 300, 1
    rng = np.random.default_rng(80)
    cb = (rng.standard_normal((Hkv, 2, R, 64, 64), dtype=np.float32) * np.float32(0.5)).astype(np.float16)
    idx = rng.integers(0, 64, size=(Hkv, R, n, 2)).astype(np.uint8)
    od = oracle.dims(1, 4 * Hkv, Hkv, R, n_groups=2, n_codes=64)
    x = oracle.decode(od, cb, idx, n).astype(np.float16)  # exact: one fp16 codeword per group
    d = vq.make_dims(1, 4 * Hkv, Hkv, R, "float16", n_groups=2, n_codes=64)
    big = torch.full((Hkv, 1, n + 9), 0x5A5A5A5A, dtype=torch.int32, device="cuda")  # one word plane at R = 1
    vq.encode_greedy(d, torch.from_numpy(x).cuda(), torch.from_numpy(cb).cuda(), codes=big, first_row=5)
    torch.cuda.synchronize()
    out = big.cpu().numpy()
    got = oracle.unpack_bits(od, np.ascontiguousarray(out[:, :, 5:5 + n]).view(np.uint32), n)
    np.testing.assert_array_equal(got, idx)
    assert np.all(out[:, :, :5] == 0x5A5A5A5A) and np.all(out[:, :, 5 + n:] == 0x5A5A5A5A)


def test_pages_attn_sixteen_kv_heads(vq):
    announce("attn_decode bit-packed 16 KV heads, R=11")
    cfg = pages_cfg("pages_kv16", 3, (5000, 1, 2049), 11, 95, n_kv=16)
    check_attn(vq, cfg, workloads.make_inputs(cfg))


@pytest.mark.parametrize("packed", [False, True])
def test_encode_then_attend_round_trip(vq, packed):
    # keys and values encoded on the GPU into the cache layout, then read by the attention kernel: the output
    # matches the oracle's attention over the same stored codes (written by one kernel, read by another)
    announce(f"encode -> attn_decode round trip, {'bit-packed R=11' if packed else 'byte R=2'}")
    Hkv, L = 2, 3000
    G, N, R = (2, 64, 11) if packed else (16, 256, 2)
    W = 128 // G
    cfg = workloads.custom("roundtrip", 1, 4 * Hkv, Hkv, (L,), R, "float16", 97, n_groups=G, n_codes=N)
    inp = workloads.make_inputs(cfg)
    rng = np.random.default_rng(98)
    xk = (rng.standard_normal((Hkv, L, 128), dtype=np.float32) * np.float32(0.8)).astype(np.float16)
    xv = (rng.standard_normal((Hkv, L, 128), dtype=np.float32) * np.float32(0.8)).astype(np.float16)
    d = vq.dims_of(cfg)
    kc = vq.encode_greedy(d, torch.from_numpy(xk).cuda(), torch.from_numpy(inp["k_cb"]).cuda())
    vc = vq.encode_greedy(d, torch.from_numpy(xv).cuda(), torch.from_numpy(inp["v_cb"]).cuda())
    torch.cuda.synchronize()
    kc, vc = kc.cpu().numpy(), vc.cpu().numpy()
    if packed:
        kc, vc = kc.view(np.uint32), vc.view(np.uint32)
    assert W * G == 128
    check_attn(vq, cfg, dict(inp, k_codes=kc, v_codes=vc))
