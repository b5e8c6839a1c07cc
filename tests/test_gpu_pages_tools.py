"""GPU parity of the codebook tools on the bit-packed layout (one 6-bit index per 64 dims, N = 64, R up to 32).

The q x codebook table, the value reduction through code bins and the codebook M-step, each against the
fp64 oracle on the same inputs; bit-packed records are built by workloads.pack_bits and unpacked for the
oracle by oracle_unpack_bits (both pinned against a big-integer bitstream on the CPU).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("R", [1, 11, 32])
def test_pages_qcodebook_table_matches_oracle(vq, R):
    announce(f"qcodebook_table bit-packed R={R}")
    cfg = pages_cfg("tab", 2, (5, 5), R, 90 + R)
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    got = vq.qcodebook_table(d, torch.from_numpy(inp["q"]).cuda(), torch.from_numpy(inp["k_cb"]).cuda())
    torch.cuda.synchronize()
    assert tuple(got.shape) == (2, 8, 2, R, 64, 64)
    ref = oracle.table(oracle.dims_of(cfg), inp["q"], inp["k_cb"])
    g = got.float().cpu().numpy().astype(np.float64)
    # each entry is an fp32 product pair rounded once to fp16
    for b in range(2):
        for h in range(8):
            err = np.abs(g[b, h] - ref[b, h]).max() / np.abs(ref[b, h]).max()
            assert err <= 1e-3, (b, h, err)


@pytest.mark.parametrize("R,signed", [(1, False), (5, True), (8, False), (11, "mixed"), (21, False), (32, True),
                                      (32, False)])
def test_pages_value_reduce_matches_oracle(vq, R, signed):
    """Weights of either sign; "mixed": negative only in a few tokens of the second 2048-token split of the first
    sequence (one workgroup takes the signed bins, the others the non-negative ones)."""
    announce(f"value_reduce bit-packed R={R} signed={signed}")
    cfg = pages_cfg("vr", 3, (2500, 1, 1024), R, 100 + R)
    inp = workloads.make_inputs(cfg)
    L = int(inp["max_len"])
    T = int(inp["total_tokens"])
    rng = np.random.default_rng(110 + R)
    p = rng.uniform(-1 if signed is True else 0, 1, size=(3, 8, L)).astype(np.float32)
    if signed == "mixed":
        p[0, 5, 2200:2203] *= -1.0
    d = vq.dims_of(cfg)
    v_words = torch.from_numpy(np.ascontiguousarray(inp["v_codes"]).view(np.int32)).cuda()
    got = vq.value_reduce(d, torch.from_numpy(p).cuda(), v_words, torch.from_numpy(inp["v_cb"]).cuda(),
                          torch.from_numpy(inp["seq_start"]).cuda(), torch.from_numpy(inp["seq_len"]).cuda(), L, T)
    torch.cuda.synchronize()
    od = oracle.dims_of(cfg)
    vc = oracle.unpack_bits(od, inp["v_codes"], T)
    ref = oracle.value_reduce(od, p, vc, inp["v_cb"], inp["seq_start"], inp["seq_len"], L)
    err = rowwise_rel_err(got.cpu().numpy(), ref)
    print(f"value_reduce bit-packed R={R}: {err:.3e}", flush=True)
    assert err <= 2e-3


def pages_fit_inputs(Hkv, n, R, seed):
    rng = np.random.default_rng(seed)
    cb = (rng.standard_normal((Hkv, 2, R, 64, 64), dtype=np.float32) * np.float32(0.5)).astype(np.float16)
    x = (rng.standard_normal((Hkv, n, 128), dtype=np.float32) * np.float32(0.7)).astype(np.float16)
    return x, cb


@pytest.mark.parametrize("R,n", [(1, 3000), (11, 2500), (32, 1001)])
def test_pages_codebook_update_matches_oracle(vq, R, n):
    """The M-step on bit-packed records against the oracle's for the same assignment (codes 60..63 unused)."""
    announce(f"codebook_update bit-packed R={R} n={n}")
    Hkv = 2
    x, cb = pages_fit_inputs(Hkv, n, R, 120 + R)
    rng = np.random.default_rng(130 + R)
    codes = rng.integers(0, 60, size=(Hkv, R, n, 2)).astype(np.uint8)
    words = workloads.pack_bits(codes, 6)
    d = vq.make_dims(1, 4 * Hkv, Hkv, R, "float16", n_groups=2, n_codes=64)
    args = (torch.from_numpy(x).cuda(), torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).cuda(),
            torch.from_numpy(cb).cuda())
    got = vq.codebook_update(d, *args)
    again = vq.codebook_update(d, *args)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    np.testing.assert_array_equal(again.cpu().numpy(), got)  # exact sums: no dependence on the order of adds
    od = oracle.dims(1, 4 * Hkv, Hkv, R, n_groups=2, n_codes=64)
    np.testing.assert_array_equal(oracle.unpack_bits(od, words, n), codes)  # the records hold these codes
    ref, counts = oracle.codebook_update(od, x, cb, codes, want_counts=True)
    used = counts > 0
    assert not used[..., 60:].any()
    np.testing.assert_array_equal(got[..., 60:, :], cb[..., 60:, :])  # unused codewords are kept
    np.testing.assert_array_equal(got[~used], cb[~used])
    # fp64 residuals summed exactly, rounded to fp16 at the end: within one fp16 ulp of the fp64 mean
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)


def test_pages_fit_codebook_r1_error_never_increases(vq):
    """E-step (encode_greedy) + M-step (codebook_update) on bit-packed records at R = 1 is Lloyd's iteration on
    64-dim groups: the squared error, measured by the oracle's decode of the unpacked codes, does not increase
    (beyond the fp16 rounding of the codewords, a second-order effect: 1e-4 relative is allowed)."""
    announce("fit_codebook bit-packed R=1")
    Hkv, n, R = 1, 4000, 1
    rng = np.random.default_rng(140)
    x = (rng.standard_normal((Hkv, n, 128), dtype=np.float32) * np.float32(0.7)).astype(np.float16)
    pick = rng.choice(n, size=64, replace=False)  # initial codewords are data points
    cb = np.stack([np.stack([x[0, pick, 64 * g:64 * (g + 1)] for g in range(2)])])[:, :, None].copy()
    d = vq.make_dims(1, 4, Hkv, R, "float16", n_groups=2, n_codes=64)
    od = oracle.dims(1, 4, Hkv, R, n_groups=2, n_codes=64)
    xt, cur = torch.from_numpy(x).cuda(), torch.from_numpy(cb).cuda()
    errs = []
    for _ in range(5):
        cur_np = cur.cpu().numpy()
        cur, words = vq.fit_codebook(d, xt, cur, 1)
        torch.cuda.synchronize()
        codes = oracle.unpack_bits(od, words.cpu().numpy().view(np.uint32), n)
        errs.append(float(((x.astype(np.float64) - oracle.decode(od, cur_np, codes, n)) ** 2).sum()))
    print("fit errors", errs, flush=True)
    assert all(b <= a * (1 + 1e-4) for a, b in zip(errs, errs[1:]))
    assert errs[-1] < 0.95 * errs[0]
