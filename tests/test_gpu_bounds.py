"""GPU: sequence descriptors outside their documented bounds are clamped by the kernels.

seq_start and seq_len live in device memory, so the host cannot check them. Each kernel clamps them:
the start into [0, total_tokens], the length into [0, min(max_len, total_tokens - start)]. These tests
pass descriptors that break each bound and compare with the oracle run on the clamped descriptors.

Every buffer the kernels read is padded on both sides (codes, RoPE table, weights, workspace), so even
an unclamped read would stay inside memory these tests allocated.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"float16": 2e-3, "float32": 1e-5}
LENGTHS = (3000, 700, 1500, 200)  # natural layout: starts 0, 3000, 3700, 5200; 5400 rows
MAX_LEN = 3000
PAD = 1 << 20  # bytes on each side of every padded buffer
# (start, length) as passed on the device, and the clamped pair the kernels must use
PASSED = [(0, 3500), (-100, 700), (3700, 11500), (5500, 200)]  # past max_len, negative start, past the rows,
CLAMPED = [(0, 3000), (0, 700), (3700, 1700), (0, 0)]          # start past the rows
ROPE_POSITIONS = 16384


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


def padded(arr, keep):
    """Device copy of arr inside a zero buffer with PAD bytes before and after; returns a typed view."""
    a = np.ascontiguousarray(arr)
    raw = torch.from_numpy(a.reshape(-1).view(np.uint8).copy())
    buf = torch.zeros(PAD + raw.numel() + PAD, dtype=torch.uint8, device="cuda")
    buf[PAD:PAD + raw.numel()] = raw.cuda()
    keep.append(buf)
    tdt = {np.dtype(np.uint8): torch.uint8, np.dtype(np.uint32): torch.int32, np.dtype(np.float32): torch.float32}
    return buf[PAD:PAD + raw.numel()].view(tdt[a.dtype])


def descriptors(pairs):
    start = np.array([s for s, _ in pairs], dtype=np.int64)
    length = np.array([n for _, n in pairs], dtype=np.int32)
    return start, length


CASES = [("byte_f16_r2", dict(n_residuals=2, dtype="float16")),
         ("byte_f32_r1", dict(n_residuals=1, dtype="float32")),
         ("packed_f16_r11", dict(n_residuals=11, dtype="float16", n_groups=2, n_codes=64))]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_attn_decode_clamps_sequence_descriptors(vq, name, kw):
    announce(f"attn_decode out-of-bounds descriptors {name}")
    R, dtype = kw["n_residuals"], kw["dtype"]
    extra = {k: v for k, v in kw.items() if k in ("n_groups", "n_codes")}
    cfg = workloads.custom(f"bounds_{name}", len(LENGTHS), 8, 2, LENGTHS, R, dtype, 31, **extra)
    inp = workloads.make_inputs(cfg)
    total = int(inp["total_tokens"])
    d = vq.dims_of(cfg)
    tdt = torch.float16 if dtype == "float16" else torch.float32
    keep = []
    k_codes, v_codes = padded(inp["k_codes"], keep), padded(inp["v_codes"], keep)
    q = torch.from_numpy(inp["q"]).cuda()
    k_cb = torch.from_numpy(inp["k_cb"]).cuda().to(tdt)
    v_cb = torch.from_numpy(inp["v_cb"]).cuda().to(tdt)
    rope = vq.rope_table(d, ROPE_POSITIONS)
    need = vq.attn_decode_workspace_size(d, MAX_LEN)
    ws = torch.zeros(4 * need + PAD, dtype=torch.uint8, device="cuda")
    s_pass, l_pass = descriptors(PASSED)
    got = vq.attn_decode(d, q, k_codes, v_codes, k_cb, v_cb, torch.from_numpy(s_pass).cuda(),
                         torch.from_numpy(l_pass).cuda(), MAX_LEN, total, rope, ROPE_POSITIONS, ws).clone()
    # a call within bounds on the same workspace: its arrival counters must have been left at zero
    nat = vq.attn_decode(d, q, k_codes, v_codes, k_cb, v_cb, torch.from_numpy(inp["seq_start"]).cuda(),
                         torch.from_numpy(inp["seq_len"]).cuda(), MAX_LEN, total, rope, ROPE_POSITIONS, ws).clone()
    torch.cuda.synchronize()
    kc, vc = inp["k_codes"], inp["v_codes"]
    od = oracle.dims_of(cfg)
    if cfg.packed:
        kc, vc = oracle.unpack_bits(od, kc, total), oracle.unpack_bits(od, vc, total)
    s_cl, l_cl = descriptors(CLAMPED)
    ref = oracle.attn_decode(od, inp["q"], kc, vc, inp["k_cb"], inp["v_cb"], s_cl, l_cl, MAX_LEN, n_threads=16)
    ref_nat = oracle.attn_decode(od, inp["q"], kc, vc, inp["k_cb"], inp["v_cb"], inp["seq_start"], inp["seq_len"],
                                 MAX_LEN, n_threads=16)
    g = got.cpu().numpy()
    assert np.all(g[3] == 0.0)  # start past the rows: an empty sequence
    err = rowwise_rel_err(g[:3], ref[:3])
    err_nat = rowwise_rel_err(nat.cpu().numpy(), ref_nat)
    print(f"{name}: clamped {err:.3e}, following call {err_nat:.3e}", flush=True)
    assert err <= TOL[dtype]
    assert err_nat <= TOL[dtype]


@pytest.mark.parametrize("dtype,R,packed", [("float16", 2, False), ("float32", 1, False), ("float16", 21, True)])
def test_value_reduce_clamps_sequence_descriptors(vq, dtype, R, packed):
    announce(f"value_reduce out-of-bounds descriptors {dtype} R={R} packed={packed}")
    extra = dict(n_groups=2, n_codes=64) if packed else {}
    cfg = workloads.custom("bounds_vr", len(LENGTHS), 8, 2, LENGTHS, R, dtype, 32, **extra)
    inp = workloads.make_inputs(cfg)
    total = int(inp["total_tokens"])
    d = vq.dims_of(cfg)
    tdt = torch.float16 if dtype == "float16" else torch.float32
    keep = []
    rng = np.random.default_rng(33)
    p = rng.uniform(0, 1, size=(len(LENGTHS), 8, MAX_LEN)).astype(np.float32)
    v_codes = padded(inp["v_codes"], keep)
    v_cb = torch.from_numpy(inp["v_cb"]).cuda().to(tdt)
    ws = torch.zeros(4 * vq.value_reduce_workspace_size(d, MAX_LEN) + PAD, dtype=torch.uint8, device="cuda")
    s_pass, l_pass = descriptors(PASSED)
    got = vq.value_reduce(d, padded(p, keep), v_codes, v_cb, torch.from_numpy(s_pass).cuda(),
                          torch.from_numpy(l_pass).cuda(), MAX_LEN, total, ws)
    torch.cuda.synchronize()
    s_cl, l_cl = descriptors(CLAMPED)
    od = oracle.dims_of(cfg)
    vc = oracle.unpack_bits(od, inp["v_codes"], total) if packed else inp["v_codes"]
    ref = oracle.value_reduce(od, p, vc, inp["v_cb"], s_cl, l_cl, MAX_LEN)
    g = got.cpu().numpy()
    assert np.all(g[3] == 0.0)
    err = rowwise_rel_err(g[:3], ref[:3])
    print(f"value_reduce {dtype} R={R}: {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("packed", [False, True])
def test_all_sequences_empty(vq, packed):
    """max_len = 0 and total_tokens = 0: no code row is read and every output row is zero."""
    announce(f"all sequences empty packed={packed}")
    extra = dict(n_groups=2, n_codes=64) if packed else {}
    R = 11 if packed else 2
    cfg = workloads.custom("empty", 3, 8, 2, (0, 0, 0), R, "float16", 34, **extra)
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    codes = torch.zeros(4096, dtype=torch.int32, device="cuda")  # never read
    q = torch.from_numpy(inp["q"]).cuda()
    k_cb, v_cb = torch.from_numpy(inp["k_cb"]).cuda(), torch.from_numpy(inp["v_cb"]).cuda()
    s0 = torch.zeros(3, dtype=torch.int64, device="cuda")
    l0 = torch.zeros(3, dtype=torch.int32, device="cuda")
    rope = vq.rope_table(d, 1)
    out = torch.full((3, 8, 128), 7.0, device="cuda")
    vq.attn_decode(d, q, codes, codes, k_cb, v_cb, s0, l0, 0, 0, rope, 1, out=out)
    p = torch.zeros(16, dtype=torch.float32, device="cuda")
    vr = torch.full((3, 8, 128), 7.0, device="cuda")
    vq.value_reduce(d, p, codes, v_cb, s0, l0, 0, 0, out=vr)
    torch.cuda.synchronize()
    assert torch.all(out == 0.0) and torch.all(vr == 0.0)
