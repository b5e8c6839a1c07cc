"""Calls on a non-default stream, with the binding allocating the workspace and outputs.

The binding allocates temporaries (the zero-filled attention workspace, the value-reduce partials) and outputs
with the launch stream current, so the zero fill runs on that stream ahead of the kernel and a freed temporary
is reused only by later work on the same stream. Here the current stream is kept busy with a long matmul while
each call goes to a side stream: a workspace zeroed on the busy stream would still hold stale bytes when the
kernel starts. Results must equal the default-stream results bit for bit (same kernels, same inputs).
"""
import sys

import numpy as np
import pytest

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


def busy_current_stream():
    """Queue a few milliseconds of work on the current stream; returns the tensors so they outlive the call."""
    a = torch.randn(4096, 4096, device="cuda")
    outs = [a @ a for _ in range(6)]
    return a, outs


def poison_pool(nbytes):
    """Leave freed blocks full of 0xff in the side stream's pool, so a workspace that were not zeroed on that
    stream before the kernel would start with non-zero arrival counters."""
    junk = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    del junk


CASES = [
    ("byte_f16_r2", workloads.custom("st_b16", 2, 32, 8, (6000, 17000), 2, "float16", 81)),
    ("bit_packed_r11", workloads.custom("st_g64", 2, 32, 8, (9000, 4000), 11, "float16", 82, n_groups=2,
                                        n_codes=64)),
]


@pytest.mark.parametrize("name,cfg", CASES)
def test_attn_decode_on_side_stream(vq, name, cfg):
    announce(f"attn_decode on a side stream: {name}")
    inp = workloads.make_inputs(cfg)
    d = vq.dims_of(cfg)
    layer = vq.Layer(d, inp)
    ref = layer.attn_decode().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        poison_pool(4 * vq.attn_decode_workspace_size(d, layer.max_len) + (1 << 20))
    keep = busy_current_stream()
    got = vq.attn_decode(d, layer.q, layer.k_codes, layer.v_codes, layer.k_cb, layer.v_cb, layer.seq_start,
                         layer.seq_len, layer.max_len, layer.total_tokens, layer.rope, layer.rope_positions,
                         stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    del keep
    assert torch.equal(got, ref)


def test_value_reduce_on_side_stream(vq):
    announce("value_reduce on a side stream")
    cfg = workloads.custom("st_vr", 3, 8, 2, (2500, 1, 1024), 2, "float32", 83)
    inp = workloads.make_inputs(cfg)
    L = int(inp["max_len"])
    p = torch.from_numpy(np.random.default_rng(84).uniform(0, 1, size=(3, 8, L)).astype(np.float32)).cuda()
    args = (torch.from_numpy(inp["v_codes"]).cuda(), torch.from_numpy(inp["v_cb"]).cuda(),
            torch.from_numpy(inp["seq_start"]).cuda(), torch.from_numpy(inp["seq_len"]).cuda(), L,
            int(inp["total_tokens"]))
    d = vq.dims_of(cfg)
    ref = vq.value_reduce(d, p, *args).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    keep = busy_current_stream()
    got = vq.value_reduce(d, p, *args, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    del keep
    assert torch.equal(got, ref)
