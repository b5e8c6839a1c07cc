"""Decode attention captured in a HIP graph (torch.cuda.graph) and replayed.

The entry points launch their kernels on the caller's stream and record nothing else: the attention workspace's
arrival counters (and the allocation-free entry point's static counters) are reset by the kernels themselves, so
no memset is captured. Each graph is replayed several times, with eager work and synchronizations between the
replays; every replay must equal the eager result bit for bit (same kernels, same inputs, a fixed order of
operations), and a replay after the query is rewritten in place must equal the eager result for the new query.
"""
import sys

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    ("byte_f16_r2", workloads.custom("graph_b16", 2, 8, 2, (3000, 777), 2, "float16", 61)),
    ("byte_f32_r1", workloads.custom("graph_b32", 1, 8, 2, (2500,), 1, "float32", 62)),
    ("bit_packed_r11", workloads.custom("graph_p11", 2, 8, 2, (2100, 4096), 11, "float16", 63, n_groups=2, n_codes=64)),
]


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


def capture(fn):
    """fn once on a side stream (as torch asks before a capture), then captured into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def check_replays(vq, cfg, launch, out, layer):
    """Replays of `launch` captured in a graph against eager launches of the same call."""
    launch()
    torch.cuda.synchronize()
    eager = out.clone()
    g = capture(launch)
    other = vq.Layer(vq.dims_of(cfg), workloads.make_inputs(cfg, seed=cfg.seed + 7))
    for rep in range(3):
        out.fill_(float("nan"))  # the replay must write every output
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager result"
        other.attn_decode()  # eager work between the replays
        torch.cuda.synchronize()
    # a new query in the captured buffer: the replay reads it
    layer.q.copy_(torch.flip(layer.q, dims=[1]))
    launch()
    torch.cuda.synchronize()
    layer_eager = out.clone()
    assert not torch.equal(layer_eager, eager)
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, layer_eager)
    assert np.all(np.isfinite(out.cpu().numpy()))


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_attn_decode_graph_replays(vq, name, cfg):
    announce(f"graph replay attn_decode {name}")
    layer = vq.Layer(vq.dims_of(cfg), workloads.make_inputs(cfg))
    check_replays(vq, cfg, layer.attn_decode, layer.out, layer)


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_attn_decode_noalloc_graph_replays(vq, name, cfg):
    announce(f"graph replay attn_decode_noalloc {name}")
    layer = vq.Layer(vq.dims_of(cfg), workloads.make_inputs(cfg))
    d = vq.dims_of(cfg)

    def launch():
        vq.attn_decode_noalloc(d, layer.q, layer.k_codes, layer.v_codes, layer.k_cb, layer.v_cb, layer.seq_start,
                               layer.seq_len, layer.max_len, layer.total_tokens, layer.rope, layer.rope_positions,
                               layer.out)
    check_replays(vq, cfg, launch, layer.out, layer)
