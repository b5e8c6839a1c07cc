"""commvq_attn_decode_noalloc (static device scratch, no workspace) against commvq_attn_decode.

Both entry points run the same kernels on the same inputs; only where the split partials and arrival counters
live differs. Each call is compared with the workspace entry point's output at the parity tolerance (per
(b, q head) row, max |a - b| / max |b|: 2e-3 fp16, 1e-5 fp32). Two calls in a row go through the static
scratch, the second with a smaller input (fewer sequences, KV heads and tokens), so the second call finds the
first one's partials in the array and counters that the first call must have left zero.
"""
import sys

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"float16": 2e-3, "float32": 1e-5}


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vector_quantized_kv_amd as m
    m.lib()
    return m


def rowwise_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).reshape(-1, ref.shape[-1]).max(-1)
    den = np.abs(ref).reshape(-1, ref.shape[-1]).max(-1)
    den = np.where(den == 0, 1.0, den)
    return (num / den).max()


def both(vq, cfg):
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    layer = vq.Layer(d, inp)
    ref = layer.attn_decode().clone()
    out = torch.full_like(ref, float("nan"))
    vq.attn_decode_noalloc(d, layer.q, layer.k_codes, layer.v_codes, layer.k_cb, layer.v_cb, layer.seq_start,
                           layer.seq_len, layer.max_len, layer.total_tokens, layer.rope, layer.rope_positions, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


CASES = [
    # (first call, second smaller call)
    ("byte_f16", workloads.custom("na_big", 2, 32, 8, (9000, 20000), 2, "float16", 71),
     workloads.custom("na_small", 1, 8, 2, (3000,), 1, "float16", 72)),
    ("byte_f32", workloads.custom("na_big32", 2, 8, 2, (5000, 2500), 2, "float32", 73),
     workloads.custom("na_small32", 1, 4, 1, (700,), 1, "float32", 74)),
    ("bit_packed", workloads.custom("na_bigp", 2, 32, 8, (7000, 12000), 11, "float16", 75, n_groups=2, n_codes=64),
     workloads.custom("na_smallp", 1, 8, 2, (2000,), 5, "float16", 76, n_groups=2, n_codes=64)),
]


@pytest.mark.parametrize("name,big,small", CASES)
def test_noalloc_matches_workspace_entry_point(vq, name, big, small):
    for cfg in (big, small):
        print(f"\n[case] noalloc {name}: {cfg.name} B={cfg.batch} Hkv={cfg.n_kv_heads} lengths={cfg.lengths}",
              flush=True)
        sys.stdout.flush()
        got, ref = both(vq, cfg)
        assert np.all(np.isfinite(got))
        err = rowwise_rel_err(got, ref)
        print(f"  max row-relative difference {err:.3e}; bit-identical: {bool(np.array_equal(got, ref))}", flush=True)
        assert err <= TOL[cfg.dtype]


def test_noalloc_rejects_oversized_calls(vq):
    # 17 x 1024 (sequence, KV head) pairs: more arrival counters than the static scratch holds; rejected on the
    # host before any launch (the pointers are never read)
    d = vq.make_dims(1024, 68, 17, 2)
    fake = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = vq.lib().commvq_attn_decode_noalloc(
        vq.ctypes.byref(d), *([vq.ctypes.c_void_p(fake.data_ptr())] * 7), 100, 100,
        vq.ctypes.c_void_p(fake.data_ptr()), 100, vq.ctypes.c_void_p(fake.data_ptr()), None)
    assert st in (vq.EUNSUPPORTED,), st
    # 64 sequences of 64K tokens: partials of about 16 MiB, beyond the 8 MiB static scratch; rejected on the host
    d = vq.make_dims(64, 32, 8, 2)
    assert vq.attn_decode_workspace_size(d, 65536) > (8 << 20)
    st = vq.lib().commvq_attn_decode_noalloc(
        vq.ctypes.byref(d), *([vq.ctypes.c_void_p(fake.data_ptr())] * 7), 65536, 64 * 65536,
        vq.ctypes.c_void_p(fake.data_ptr()), 65536, vq.ctypes.c_void_p(fake.data_ptr()), None)
    assert st == vq.EWORKSPACE, st
    assert "scratch" in vq.last_error_detail()
