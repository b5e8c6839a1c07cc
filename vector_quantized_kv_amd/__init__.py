"""Python binding of libcommvq (CommVQ decode-step attention on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C ABI
declared in include/commvq.h. torch supplies device memory and the current HIP stream. There is no
CPU fallback: if libcommvq.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# COMMVQ_LIBRARY names another build of the same C ABI (the host-only sanitizer build, which has no device
# code and fails every launch with COMMVQ_EHIP); by default the in-tree libcommvq.so is loaded.
LIB_PATH = os.environ.get("COMMVQ_LIBRARY") or os.path.join(PKG, "libcommvq.so")

F16, F32 = 1, 2
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4

EXPORTED_SYMBOLS = (
    "commvq_status_string", "commvq_last_error_detail", "commvq_rope_table_size", "commvq_rope_table",
    "commvq_qcodebook_table", "commvq_attn_decode_workspace_size", "commvq_attn_decode",
    "commvq_value_reduce_workspace_size", "commvq_value_reduce", "commvq_encode_greedy", "commvq_codebook_update",
    "commvq_debug_unpack", "commvq_attn_decode_noalloc",
)


class CommVQError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {detail}")
        self.status = status


class Dims(ctypes.Structure):
    """Mirror of commvq_dims."""
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_groups", ctypes.c_int32), ("n_residuals", ctypes.c_int32),
                ("n_codes", ctypes.c_int32), ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


def make_dims(batch, n_q_heads, n_kv_heads, n_residuals, dtype="float16", head_dim=128, n_groups=16,
              n_codes=256, rope_base=500000.0, softmax_scale=None) -> Dims:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    dt = {"float16": F16, "float32": F32, F16: F16, F32: F32}[dtype]
    return Dims(batch, n_q_heads, n_kv_heads, head_dim, n_groups, n_residuals, n_codes, rope_base, softmax_scale, dt)


def dims_of(cfg) -> Dims:
    """Dims of a workloads.Config-like object."""
    return make_dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_residuals, cfg.dtype, cfg.head_dim,
                     cfg.n_groups, cfg.n_codes, cfg.rope_base, cfg.softmax_scale)


_lib = None


def lib():
    """Load libcommvq.so (built in-tree by vector_quantized_kv_amd.build). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m vector_quantized_kv_amd.build` "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, D = ctypes.c_void_p, ctypes.POINTER(Dims)
        i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.commvq_status_string.argtypes, L.commvq_status_string.restype = [ctypes.c_int], ctypes.c_char_p
        L.commvq_last_error_detail.argtypes, L.commvq_last_error_detail.restype = [], ctypes.c_char_p
        L.commvq_rope_table_size.argtypes, L.commvq_rope_table_size.restype = [D, i32], sz
        L.commvq_rope_table.argtypes, L.commvq_rope_table.restype = [D, i32, P, sz, P], ctypes.c_int
        L.commvq_qcodebook_table.argtypes, L.commvq_qcodebook_table.restype = [D, P, P, P, P], ctypes.c_int
        L.commvq_attn_decode_workspace_size.argtypes, L.commvq_attn_decode_workspace_size.restype = [D, i32], sz
        L.commvq_attn_decode.argtypes = [D, P, P, P, P, P, P, P, i32, i64, P, i32, P, sz, P, P]
        L.commvq_attn_decode.restype = ctypes.c_int
        L.commvq_attn_decode_noalloc.argtypes = [D, P, P, P, P, P, P, P, i32, i64, P, i32, P, P]
        L.commvq_attn_decode_noalloc.restype = ctypes.c_int
        L.commvq_value_reduce_workspace_size.argtypes, L.commvq_value_reduce_workspace_size.restype = [D, i32], sz
        L.commvq_value_reduce.argtypes = [D, P, P, P, P, P, i32, i64, P, sz, P, P]
        L.commvq_value_reduce.restype = ctypes.c_int
        L.commvq_encode_greedy.argtypes = [D, P, P, i64, P, i64, i64, P]
        L.commvq_encode_greedy.restype = ctypes.c_int
        L.commvq_codebook_update.argtypes = [D, P, P, i64, P, P, P]
        L.commvq_codebook_update.restype = ctypes.c_int
        L.commvq_debug_unpack.argtypes, L.commvq_debug_unpack.restype = [D, P, i64, P, P], ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().commvq_status_string(int(status)).decode()


def last_error_detail() -> str:
    return lib().commvq_last_error_detail().decode()


def _check(status: int, where: str):
    if status != OK:
        raise CommVQError(status, where, last_error_detail())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _launch_stream(stream=None):
    """The stream a call is enqueued on: `stream`, else torch's current stream."""
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream=None):
    return ctypes.c_void_p(_launch_stream(stream).cuda_stream)


def _on(stream=None):
    """Context that makes the launch stream current while the binding allocates outputs and temporaries: the
    caching allocator then ties them to that stream (a temporary freed on return is reused only by later work
    on the same stream, which runs after the kernel), and the workspace zero-fill runs on it, ahead of the
    kernel that reads it."""
    import torch
    return torch.cuda.stream(_launch_stream(stream))


def _torch_dtype(d: Dims):
    import torch
    return torch.float16 if d.dtype == F16 else torch.float32


def rope_table(d: Dims, n_positions: int, device="cuda", stream=None, out=None):
    """Two-level RoPE phase table for positions 0 .. n_positions-1 (see commvq_rope_table); written into `out`
    (fp32, at least commvq_rope_table_size bytes) when given."""
    import torch
    nbytes = lib().commvq_rope_table_size(ctypes.byref(d), int(n_positions))
    if nbytes == 0:
        _check(lib().commvq_rope_table(ctypes.byref(d), int(n_positions), None, 0, None), "rope_table")
    if out is not None:
        if out.dtype != torch.float32 or out.numel() * 4 < nbytes:
            raise ValueError(f"rope_table: out must be fp32 with at least {nbytes // 4} elements")
        t = out
    else:
        with _on(stream):
            t = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    _check(lib().commvq_rope_table(ctypes.byref(d), int(n_positions), ctypes.c_void_p(t.data_ptr()), nbytes,
                                   _stream(stream)), "rope_table")
    return t


def qcodebook_table(d: Dims, q, k_codebook, out=None, stream=None):
    import torch
    if out is None:
        with _on(stream):
            out = torch.empty((d.batch, d.n_q_heads, d.n_groups, d.n_residuals, d.n_codes,
                               d.head_dim // d.n_groups), dtype=_torch_dtype(d), device=q.device)
    _check(lib().commvq_qcodebook_table(ctypes.byref(d), _ptr(q), _ptr(k_codebook), _ptr(out), _stream(stream)),
           "qcodebook_table")
    return out


def attn_decode_workspace_size(d: Dims, max_len: int) -> int:
    return int(lib().commvq_attn_decode_workspace_size(ctypes.byref(d), int(max_len)))


def attn_workspace(d: Dims, max_len: int, device="cuda"):
    """Zero-filled attention workspace (its arrival counters must start at zero; calls leave them zero)."""
    import torch
    return torch.zeros(max(attn_decode_workspace_size(d, max_len), 256), dtype=torch.uint8, device=device)


def attn_decode(d: Dims, q, k_codes, v_codes, k_codebook, v_codebook, seq_start, seq_len, max_len: int,
                total_tokens: int, rope, rope_positions: int, workspace=None, out=None, stream=None):
    """Decode-step attention; returns out [B][Hq][D] fp32 (see commvq_attn_decode)."""
    import torch
    if out is None or workspace is None:
        with _on(stream):
            if out is None:
                out = torch.empty((d.batch, d.n_q_heads, d.head_dim), dtype=torch.float32, device=q.device)
            if workspace is None:
                workspace = attn_workspace(d, max_len, q.device)
    st = lib().commvq_attn_decode(ctypes.byref(d), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_codebook),
                                  _ptr(v_codebook), _ptr(seq_start), _ptr(seq_len), int(max_len), int(total_tokens),
                                  _ptr(rope), int(rope_positions), _ptr(workspace), workspace.numel() *
                                  workspace.element_size(), _ptr(out), _stream(stream))
    _check(st, "attn_decode")
    return out


def attn_decode_noalloc(d: Dims, q, k_codes, v_codes, k_codebook, v_codebook, seq_start, seq_len, max_len: int,
                        total_tokens: int, rope, rope_positions: int, out, stream=None):
    """Decode-step attention through commvq_attn_decode_noalloc (the library's static scratch; no workspace).
    `out` [B][Hq][D] fp32 must be given: nothing is allocated on this path."""
    st = lib().commvq_attn_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_codebook),
                                          _ptr(v_codebook), _ptr(seq_start), _ptr(seq_len), int(max_len),
                                          int(total_tokens), _ptr(rope), int(rope_positions), _ptr(out),
                                          _stream(stream))
    _check(st, "attn_decode_noalloc")
    return out


def value_reduce_workspace_size(d: Dims, max_len: int) -> int:
    return int(lib().commvq_value_reduce_workspace_size(ctypes.byref(d), int(max_len)))


def value_reduce(d: Dims, p, v_codes, v_codebook, seq_start, seq_len, max_len: int, total_tokens: int,
                 workspace=None, out=None, stream=None):
    """out[b][h] = sum_t p[b][h][t] * vhat_t via code bins (see commvq_value_reduce)."""
    import torch
    if out is None or workspace is None:
        with _on(stream):
            if out is None:
                out = torch.empty((d.batch, d.n_q_heads, d.head_dim), dtype=torch.float32, device=p.device)
            if workspace is None:
                workspace = torch.empty(max(value_reduce_workspace_size(d, max_len), 16), dtype=torch.uint8,
                                        device=p.device)
    st = lib().commvq_value_reduce(ctypes.byref(d), _ptr(p), _ptr(v_codes), _ptr(v_codebook), _ptr(seq_start),
                                   _ptr(seq_len), int(max_len), int(total_tokens), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream))
    _check(st, "value_reduce")
    return out


def encode_greedy(d: Dims, x, codebook, codes=None, first_row: int = 0, stream=None):
    """Greedy residual codes of x [Hkv][n][D] (see commvq_encode_greedy). With codes=None a new array is
    returned: [Hkv][R][n][G] uint8, or for the bit-packed layout the word planes [Hkv][words][n] (int32
    tensor holding the uint32 words); otherwise the tokens are written to rows first_row.. of codes."""
    import torch
    n = int(x.shape[1])
    packed = d.n_codes < 256
    if codes is None:
        with _on(stream):
            if packed:
                words = (6 * d.n_residuals * d.n_groups + 31) // 32
                codes = torch.zeros((d.n_kv_heads, words, n), dtype=torch.int32, device=x.device)
            else:
                codes = torch.zeros((d.n_kv_heads, d.n_residuals, n, d.n_groups), dtype=torch.uint8,
                                    device=x.device)
    rows = int(codes.shape[2])
    _check(lib().commvq_encode_greedy(ctypes.byref(d), _ptr(x), _ptr(codebook), n, _ptr(codes), rows,
                                      int(first_row), _stream(stream)), "encode_greedy")
    return codes


def codebook_update(d: Dims, x, codes, codebook_in, codebook_out=None, stream=None):
    """One M-step of the residual codebook fit (see commvq_codebook_update): x [Hkv][n][D], codes
    [Hkv][R][n][G] uint8 (bit-packed layout: word planes [Hkv][words][n]), codebook_in [Hkv][G][R][N][W]. Returns codebook_out (a new tensor if None)."""
    import torch
    n = int(x.shape[1])
    if codebook_out is None:
        with _on(stream):
            codebook_out = torch.empty_like(codebook_in)
    _check(lib().commvq_codebook_update(ctypes.byref(d), _ptr(x), _ptr(codes), n, _ptr(codebook_in),
                                        _ptr(codebook_out), _stream(stream)), "codebook_update")
    return codebook_out


def fit_codebook(d: Dims, x, codebook, iterations: int, stream=None):
    """Residual codebook fit on the GPU: `iterations` rounds of the E-step (commvq_encode_greedy) and the
    M-step (commvq_codebook_update), starting from `codebook`. Returns (codebook, codes of the last E-step)."""
    cur = codebook
    codes = None
    for _ in range(int(iterations)):
        codes = encode_greedy(d, x, cur, codes=codes, stream=stream)
        cur = codebook_update(d, x, codes, cur, stream=stream)
    return cur, codes


def debug_unpack(d: Dims, codes, total_tokens: int, out=None, stream=None):
    import torch
    if out is None:
        with _on(stream):
            out = torch.empty((d.n_kv_heads, d.n_residuals, int(total_tokens), d.n_groups), dtype=torch.int32,
                              device=codes.device)
    _check(lib().commvq_debug_unpack(ctypes.byref(d), _ptr(codes), int(total_tokens), _ptr(out), _stream(stream)),
           "debug_unpack")
    return out


def _code_array(a):
    import numpy as np
    a = np.ascontiguousarray(a)
    return a.view(np.int32) if a.dtype == np.uint32 else a


class Layer:
    """Device-resident inputs of one decode step for one layer (helper for tests and benchmarks)."""

    def __init__(self, d: Dims, inputs: dict, device="cuda", rope=None, rope_positions=None):
        import torch
        self.d = d
        dt = _torch_dtype(d)
        self.q = torch.from_numpy(inputs["q"]).to(device=device, dtype=dt)
        self.k_cb = torch.from_numpy(inputs["k_cb"]).to(device=device, dtype=dt)
        self.v_cb = torch.from_numpy(inputs["v_cb"]).to(device=device, dtype=dt)
        # bit-packed word planes (uint32 words) travel as int32 tensors of the same bits
        self.k_codes = torch.from_numpy(_code_array(inputs["k_codes"])).to(device)
        self.v_codes = torch.from_numpy(_code_array(inputs["v_codes"])).to(device)
        self.seq_start = torch.from_numpy(inputs["seq_start"]).to(device)
        self.seq_len = torch.from_numpy(inputs["seq_len"]).to(device)
        self.max_len = int(inputs["max_len"])
        self.total_tokens = int(inputs["total_tokens"])
        self.rope_positions = rope_positions if rope_positions is not None else max(self.max_len, 1)
        self.rope = rope if rope is not None else rope_table(d, self.rope_positions, device=device)
        self.workspace = attn_workspace(d, self.max_len, device)
        self.out = torch.empty((d.batch, d.n_q_heads, d.head_dim), dtype=torch.float32, device=device)

    def attn_decode(self, stream=None):
        return attn_decode(self.d, self.q, self.k_codes, self.v_codes, self.k_cb, self.v_cb, self.seq_start,
                           self.seq_len, self.max_len, self.total_tokens, self.rope, self.rope_positions,
                           self.workspace, self.out, stream)
