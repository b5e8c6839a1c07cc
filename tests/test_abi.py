"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and rejects bad
arguments on the host (these calls return before any HIP call, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import vector_quantized_kv_amd as vq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols(header="commvq.h"):
    with open(os.path.join(ROOT, "include", header)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(commvq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = vq.lib()
    names = declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(vq.EXPORTED_SYMBOLS)


def test_probe_library_exports_its_header():
    """The benchmark's measurement probes live in a library of their own, not in the attention ABI."""
    from vector_quantized_kv_amd import build as vbuild
    if not os.path.exists(vbuild.PROBES_LIB):
        pytest.skip("libcommvq_probes.so not built")
    L = ctypes.CDLL(vbuild.PROBES_LIB)
    names = declared_symbols("commvq_probes.h")
    assert names == ["commvq_probe_lds_bin_add", "commvq_probe_lds_gather", "commvq_probe_read_stream"]
    for n in names:
        assert hasattr(L, n), n
        assert not hasattr(vq.lib(), n), n
    # host checks reject bad arguments before any launch
    L.commvq_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
    L.commvq_probe_lds_gather.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.commvq_probe_lds_bin_add.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert L.commvq_probe_read_stream(None, 16, 1, 0x1000, None) != 0
    assert L.commvq_probe_read_stream(0x1000, 15, 1, 0x1000, None) != 0
    assert L.commvq_probe_lds_gather(0, 1, 0x1000, None) != 0
    assert L.commvq_probe_lds_bin_add(1, 0, 0x1000, None) != 0
    assert L.commvq_probe_lds_bin_add(1, 1, None, None) != 0


def test_dims_struct_layout_matches_header():
    # int32 x7, pad, double, float, int32 -> 48 bytes with 8-byte alignment
    assert ctypes.sizeof(vq.Dims) == 48
    assert vq.Dims.rope_base.offset == 32


def test_status_strings():
    assert vq.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert vq.status_string(s) != "unknown status"


def _attn(d, **kw):
    args = dict(q=None, kc=None, vc=None, kb=None, vb=None, ss=None, sl=None, max_len=0, total=0, rope=None,
                rope_pos=0, ws=None, ws_bytes=0, out=None)
    args.update(kw)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first
    conv = lambda v: fake if v == "p" else v
    return vq.lib().commvq_attn_decode(ctypes.byref(d), *(conv(args[k]) for k in
                                       ("q", "kc", "vc", "kb", "vb", "ss", "sl")), args["max_len"], args["total"],
                                       conv(args["rope"]), args["rope_pos"], conv(args["ws"]), args["ws_bytes"],
                                       conv(args["out"]), None)


ALL = dict(q="p", kc="p", vc="p", kb="p", vb="p", ss="p", sl="p", rope="p", out="p", ws="p")


@pytest.mark.parametrize("field,value,status", [
    ("n_residuals", 3, vq.EUNSUPPORTED), ("n_residuals", 0, vq.EINVAL), ("head_dim", 64, vq.EUNSUPPORTED),
    ("n_groups", 8, vq.EUNSUPPORTED), ("n_codes", 64, vq.EUNSUPPORTED), ("n_q_heads", 30, vq.EINVAL),
    ("n_q_heads", 16, vq.EUNSUPPORTED), ("batch", 0, vq.EINVAL), ("dtype", 7, vq.EINVAL),
    ("rope_base", 0.5, vq.EINVAL), ("softmax_scale", 0.0, vq.EINVAL), ("softmax_scale", float("inf"), vq.EINVAL),
    ("softmax_scale", float("nan"), vq.EINVAL),
])
def test_bad_dims_rejected(field, value, status):
    d = vq.make_dims(1, 32, 8, 2)
    setattr(d, field, value)
    assert _attn(d, **ALL, max_len=10, total=10, rope_pos=10, ws_bytes=1 << 30) == status
    assert vq.last_error_detail() != ""


def test_null_pointer_and_sizes_rejected():
    d = vq.make_dims(1, 32, 8, 2)
    base = dict(ALL, max_len=100, total=100, rope_pos=100, ws_bytes=1 << 30)
    assert _attn(d, **dict(base, q=None)) == vq.EINVAL
    assert _attn(d, **dict(base, max_len=-1)) == vq.EINVAL
    assert _attn(d, **dict(base, total=-5)) == vq.EINVAL
    assert _attn(d, **dict(base, rope_pos=50)) == vq.EINVAL
    assert _attn(d, **dict(base, ws_bytes=16)) == vq.EWORKSPACE
    assert "workspace" in vq.last_error_detail()
    assert _attn(d, **dict(base, ws=None)) == vq.EWORKSPACE


def test_misaligned_codes_rejected():
    d = vq.make_dims(1, 32, 8, 2)
    L = vq.lib()
    p, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1001)
    st = L.commvq_attn_decode(ctypes.byref(d), p, odd, p, p, p, p, p, 10, 10, p, 10, p, 1 << 30, p, None)
    assert st == vq.EINVAL and "aligned" in vq.last_error_detail()
    # the query x codebook table moves codeword rows in 16-byte pieces
    assert L.commvq_qcodebook_table(ctypes.byref(d), p, odd, p, None) == vq.EINVAL
    assert "aligned" in vq.last_error_detail()
    assert L.commvq_qcodebook_table(ctypes.byref(d), p, p, odd, None) == vq.EINVAL


def test_workspace_sizes():
    # attention workspace: 256 B of arrival counters, then (m, l) per (sequence, q head, split) padded to
    # 256 B, then o[128] fp32 per (sequence, q head, split). fp16 splits are 512 x blocks-per-wave tokens
    # (8 waves x 64 tokens, blocks-per-wave 1..8), sized for about one work item per CU (256).
    def attn_ws(B, Hq, splits):
        items = B * Hq * splits
        return 256 + (items * 8 + 255) // 256 * 256 + items * 128 * 4
    d = vq.make_dims(2, 32, 8, 1)
    assert vq.attn_decode_workspace_size(d, 131072) == attn_ws(2, 32, 32)   # 4096-token splits
    assert vq.attn_decode_workspace_size(d, 1) == attn_ws(2, 32, 1)
    d1 = vq.make_dims(1, 32, 8, 2)
    assert vq.attn_decode_workspace_size(d1, 8192) == attn_ws(1, 32, 16)    # 512-token splits
    assert vq.attn_decode_workspace_size(d1, 131072) == attn_ws(1, 32, 32)  # 4096-token splits
    d32 = vq.make_dims(1, 4, 1, 2, dtype="float32")
    assert vq.attn_decode_workspace_size(d32, 1024) == attn_ws(1, 4, 4)     # fp32: 4 waves, 256-token splits
    assert vq.value_reduce_workspace_size(d, 4096) == 2 * 32 * 2 * 132 * 4  # 2048-token splits
    # RoPE table: fine fp32 pair-major (64 x 64 x 8 B), fine fp16 (64 x 64 x 4 B), fine fp32 group-major
    # (64 x 64 x 8 B), coarse (ceil(n/64) x 64 x 8 B)
    assert vq.lib().commvq_rope_table_size(ctypes.byref(d), 131072) == (4096 + 4096 + 2048 * 64) * 8
    assert vq.lib().commvq_rope_table_size(ctypes.byref(d), 0) == 0


def test_encode_greedy_rejects_bad_arguments_on_host():
    d = vq.make_dims(1, 32, 8, 2)
    L = vq.lib()
    p = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation or is a no-op
    assert L.commvq_encode_greedy(ctypes.byref(d), p, p, -1, p, 10, 0, None) == vq.EINVAL
    assert L.commvq_encode_greedy(ctypes.byref(d), p, p, 5, p, 10, 6, None) == vq.EINVAL   # rows 6..10 > 10
    assert L.commvq_encode_greedy(ctypes.byref(d), p, p, 5, p, 10, -1, None) == vq.EINVAL
    assert L.commvq_encode_greedy(ctypes.byref(d), None, p, 5, p, 10, 0, None) == vq.EINVAL
    assert L.commvq_encode_greedy(ctypes.byref(d), p, p, 0, p, 0, 0, None) == vq.OK         # nothing to do
    d.n_residuals = 3
    assert L.commvq_encode_greedy(ctypes.byref(d), p, p, 5, p, 10, 0, None) == vq.EUNSUPPORTED


def test_codebook_update_rejects_bad_arguments_on_host():
    d = vq.make_dims(1, 32, 8, 2)
    L = vq.lib()
    cb_bytes = 8 * 16 * 2 * 256 * 8 * 2  # fp16 codebook [Hkv][G][R][N][W]
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x100000 + cb_bytes)  # never dereferenced
    p = ctypes.c_void_p(0x1000)
    assert L.commvq_codebook_update(ctypes.byref(d), p, p, -1, a, b, None) == vq.EINVAL
    assert L.commvq_codebook_update(ctypes.byref(d), None, p, 5, a, b, None) == vq.EINVAL
    assert L.commvq_codebook_update(ctypes.byref(d), p, None, 5, a, b, None) == vq.EINVAL
    assert L.commvq_codebook_update(ctypes.byref(d), p, p, 5, None, b, None) == vq.EINVAL
    # output overlapping the input by one byte
    assert L.commvq_codebook_update(ctypes.byref(d), p, p, 5, a, ctypes.c_void_p(0x100000 + cb_bytes - 1),
                                    None) == vq.EINVAL
    assert L.commvq_codebook_update(ctypes.byref(d), p, p, 5, a, a, None) == vq.EINVAL
    d.n_residuals = 3
    assert L.commvq_codebook_update(ctypes.byref(d), p, p, 5, a, b, None) == vq.EUNSUPPORTED


def test_bit_packed_layout_checks_on_host():
    L = vq.lib()
    p = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation or sizes only
    d = vq.make_dims(1, 32, 8, 21, n_groups=2, n_codes=64)
    # accepted shapes: workspace and table sizes are reported
    assert vq.attn_decode_workspace_size(d, 4096) > 0
    assert L.commvq_rope_table_size(ctypes.byref(d), 4096) > 0
    for R, status in ((1, 0), (32, 0), (33, vq.EUNSUPPORTED), (0, vq.EINVAL)):
        dd = vq.make_dims(1, 32, 8, R, n_groups=2, n_codes=64)
        assert (L.commvq_attn_decode_workspace_size(ctypes.byref(dd), 64) > 0) == (status == 0), R
    # fp32 codebooks are not implemented for the bit-packed layout
    d32 = vq.make_dims(1, 32, 8, 11, dtype="float32", n_groups=2, n_codes=64)
    assert _attn(d32, **ALL) == vq.EUNSUPPORTED
    # the codebook tools take the bit-packed layout too; bad arguments are rejected before any launch
    assert L.commvq_qcodebook_table(ctypes.byref(d), p, p, None, None) == vq.EINVAL
    assert L.commvq_qcodebook_table(ctypes.byref(d32), p, p, p, None) == vq.EUNSUPPORTED
    vr = L.commvq_value_reduce_workspace_size(ctypes.byref(d), 64)
    assert vr > 0
    assert L.commvq_value_reduce(ctypes.byref(d), p, p, p, p, p, 64, 64, p, vr - 1, p, None) == vq.EWORKSPACE
    assert L.commvq_value_reduce(ctypes.byref(d), p, ctypes.c_void_p(0x1004), p, p, p, 64, 64, p, vr, p,
                                 None) == vq.EINVAL
    cb_bytes = 8 * 2 * 21 * 64 * 64 * 2  # fp16 codebook [Hkv][2][R][64][64]
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x100000 + cb_bytes)  # never dereferenced
    assert L.commvq_codebook_update(ctypes.byref(d), p, ctypes.c_void_p(0x1004), 5, a, b, None) == vq.EINVAL
    assert L.commvq_codebook_update(ctypes.byref(d), p, p, 5, a, ctypes.c_void_p(0x100000 + cb_bytes - 1),
                                    None) == vq.EINVAL  # overlap by one byte at the bit-packed size
    assert L.commvq_codebook_update(ctypes.byref(d32), p, p, 5, a, b, None) == vq.EUNSUPPORTED
    # the encoder writes bit-packed records too; misaligned records are rejected before any launch
    assert L.commvq_encode_greedy(ctypes.byref(d), p, p, 5, ctypes.c_void_p(0x1004), 10, 0, None) == vq.EINVAL
    assert L.commvq_encode_greedy(ctypes.byref(d), p, p, 5, p, 10, 6, None) == vq.EINVAL  # rows 6..10 > 10
    # mixed shapes stay unsupported
    for g, n in ((2, 256), (16, 64), (4, 64)):
        dd = vq.make_dims(1, 32, 8, 1, n_groups=g, n_codes=n)
        assert _attn(dd, **ALL) == vq.EUNSUPPORTED, (g, n)
    # misaligned records are rejected before any launch
    ws = vq.attn_decode_workspace_size(d, 64)
    st = _attn(d, **dict(ALL, kc=ctypes.c_void_p(0x1004), max_len=64, total=64, rope_pos=64, ws_bytes=ws))
    assert st == vq.EINVAL
