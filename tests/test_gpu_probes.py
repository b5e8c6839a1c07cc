"""The benchmark's measurement probes (libcommvq_probes.so) run through their C ABI and keep their contract:
every launch succeeds; the read and gather probes' sink, written only if the folded value equals a fixed
constant, stays untouched for these inputs (a zero-filled buffer folds to zero; the gather probe never writes
it); the bin-add probe's bins hold exactly one count per add."""
import ctypes
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probes():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vector_quantized_kv_amd import build as vbuild
    L = ctypes.CDLL(vbuild.PROBES_LIB)
    L.commvq_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
    L.commvq_probe_lds_gather.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.commvq_probe_lds_bin_add.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return L


def test_read_stream_probe(probes):
    print("\n[case] probe read stream", flush=True)
    sys.stdout.flush()
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for blocks in (1, 64, 2048):
        assert probes.commvq_probe_read_stream(buf.data_ptr(), buf.numel(), blocks, sink.data_ptr(), s) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def test_lds_gather_probe(probes):
    print("\n[case] probe LDS gather", flush=True)
    sys.stdout.flush()
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert probes.commvq_probe_lds_gather(4, 256, sink.data_ptr(), s) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def test_lds_bin_add_probe_counts_every_add(probes):
    print("\n[case] probe LDS bin add", flush=True)
    sys.stdout.flush()
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for iters, blocks in ((1, 1), (3, 300)):
        sink.zero_()
        assert probes.commvq_probe_lds_bin_add(iters, blocks, sink.data_ptr(), s) == 0
        torch.cuda.synchronize()
        assert int(sink.item()) == blocks * 8 * iters * 42 * 2 * 64
