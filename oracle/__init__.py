"""fp64 CPU oracle for CommVQ decode-step attention (ctypes front end of oracle.c).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library and never touches a GPU. Floating-point
inputs are converted to float64 exactly (float16 and float32 embed in float64 without rounding)
before the C code sees them.

Parity pins: every function here is checked in tests/test_oracle_pins.py against something other
than itself (identities the pages state, closed forms, brute force, library routines); see the
docstring of that file for which pin covers which function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# COMMVQ_ORACLE_SANITIZE=1: build and load the oracle with AddressSanitizer and UndefinedBehaviorSanitizer
# (the sanitizer runtimes must then be preloaded into the Python process)
_SANITIZE = os.environ.get("COMMVQ_ORACLE_SANITIZE") == "1"
_SAN_LIB = os.path.join(os.path.dirname(_HERE), "_build", "liboracle_san.so")
_SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build(force: bool = True, sanitize: Optional[bool] = None) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain C, fp64, pthreads), or with sanitize (default: the
    COMMVQ_ORACLE_SANITIZE setting) into _build/liboracle_san.so."""
    san = _SANITIZE if sanitize is None else sanitize
    out = _SAN_LIB if san else _LIB
    if force or not os.path.exists(out):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        tmp = out + ".tmp"
        flags = _SAN_FLAGS if san else ["-O2"]
        subprocess.check_call(["gcc", *flags, "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_groups", ctypes.c_int32), ("n_residuals", ctypes.c_int32),
                ("n_codes", ctypes.c_int32), ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build(force=False))
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        D = ctypes.POINTER(Dims)
        L.oracle_unpack.argtypes = [D, P, i64, P]
        L.oracle_decode.argtypes = [D, P, P, i64, P]
        L.oracle_rope.argtypes = [D, P, P, i64, P]
        L.oracle_key_block.argtypes = [ctypes.c_double, ctypes.c_double, P]
        L.oracle_rotation.argtypes = [ctypes.c_double, P]
        L.oracle_attn_decode.argtypes = [D, P, P, P, P, P, P, P, i64, i32, P, P, P, ctypes.c_int]
        L.oracle_table.argtypes = [D, P, P, P]
        L.oracle_scores_via_table.argtypes = [D, P, P, P, P, i64, i32, P]
        L.oracle_value_reduce.argtypes = [D, P, P, P, P, P, i64, i32, P]
        L.oracle_encode_greedy.argtypes = [D, P, P, i64, P, P]
        L.oracle_encode_eval.argtypes = [D, P, P, i64, P, P, P, P]
        L.oracle_codebook_update.argtypes = [D, P, P, P, i64, P, P]
        L.oracle_unpack_bits.argtypes = [D, P, i64, P]
        for f in ("oracle_unpack", "oracle_decode", "oracle_rope", "oracle_key_block", "oracle_rotation",
                  "oracle_attn_decode", "oracle_table", "oracle_scores_via_table", "oracle_value_reduce",
                  "oracle_encode_greedy", "oracle_encode_eval", "oracle_codebook_update",
                  "oracle_unpack_bits"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def dims(batch, n_q_heads, n_kv_heads, n_residuals, head_dim=128, n_groups=16, n_codes=256,
         rope_base=500000.0, softmax_scale=None) -> Dims:
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(head_dim)
    return Dims(batch, n_q_heads, n_kv_heads, head_dim, n_groups, n_residuals, n_codes, rope_base, softmax_scale)


def dims_of(cfg) -> Dims:
    """Dims of a workloads.Config."""
    return dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_residuals, cfg.head_dim, cfg.n_groups,
                cfg.n_codes, cfg.rope_base, cfg.softmax_scale)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8
    return a


def unpack(d: Dims, codes: np.ndarray, total_tokens: int) -> np.ndarray:
    c = _u8(codes)
    out = np.empty(c.shape, dtype=np.int32)
    lib().oracle_unpack(ctypes.byref(d), _ptr(c), int(total_tokens), _ptr(out))
    return out


def unpack_bits(d: Dims, words, total_tokens: int) -> np.ndarray:
    """Bit-packed word planes [Hkv][ceil(bits*R*G/32)][T] uint32 -> indices [Hkv][R][T][G] uint8."""
    ww = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.empty((d.n_kv_heads, d.n_residuals, int(total_tokens), d.n_groups), dtype=np.uint8)
    lib().oracle_unpack_bits(ctypes.byref(d), ww.ctypes.data_as(ctypes.c_void_p), int(total_tokens), _ptr(out))
    return out


def decode(d: Dims, codebook, codes, total_tokens: int) -> np.ndarray:
    cb, c = _f64(codebook), _u8(codes)
    out = np.empty((d.n_kv_heads, int(total_tokens), d.head_dim), dtype=np.float64)
    lib().oracle_decode(ctypes.byref(d), _ptr(cb), _ptr(c), int(total_tokens), _ptr(out))
    return out


def rope(d: Dims, x, pos) -> np.ndarray:
    xx = _f64(x).reshape(-1, d.head_dim)
    pp = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(-1))
    assert pp.shape[0] == xx.shape[0]
    out = np.empty_like(xx)
    lib().oracle_rope(ctypes.byref(d), _ptr(xx), _ptr(pp), xx.shape[0], _ptr(out))
    return out.reshape(np.shape(x))


def key_block(a: float, b: float) -> np.ndarray:
    m = np.empty(4, dtype=np.float64)
    lib().oracle_key_block(float(a), float(b), _ptr(m))
    return m.reshape(2, 2)


def rotation(phi: float) -> np.ndarray:
    m = np.empty(4, dtype=np.float64)
    lib().oracle_rotation(float(phi), _ptr(m))
    return m.reshape(2, 2)


def attn_decode(d: Dims, q, k_codes, v_codes, k_cb, v_cb, seq_start, seq_len, max_len: Optional[int] = None,
                n_threads: int = 1, want_scores: bool = False, want_p: bool = False):
    """Decode-step attention. Returns out [B][Hq][D] float64, plus (scores, p) [B][Hq][max_len] if asked."""
    qq, kc, vc = _f64(q), _u8(k_codes), _u8(v_codes)
    kb, vb = _f64(k_cb), _f64(v_cb)
    ss = np.ascontiguousarray(seq_start, dtype=np.int64)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    total = kc.shape[2]
    if max_len is None:
        max_len = int(sl.max()) if sl.size else 0
    out = np.empty((d.batch, d.n_q_heads, d.head_dim), dtype=np.float64)
    scores = np.empty((d.batch, d.n_q_heads, max_len), dtype=np.float64) if want_scores else None
    p = np.empty((d.batch, d.n_q_heads, max_len), dtype=np.float64) if want_p else None
    lib().oracle_attn_decode(ctypes.byref(d), _ptr(qq), _ptr(kc), _ptr(vc), _ptr(kb), _ptr(vb), _ptr(ss), _ptr(sl),
                             int(total), int(max_len), _ptr(out), _ptr(scores) if scores is not None else None,
                             _ptr(p) if p is not None else None, int(n_threads))
    if want_scores or want_p:
        return out, scores, p
    return out


def table(d: Dims, q, k_cb) -> np.ndarray:
    qq, kb = _f64(q), _f64(k_cb)
    W = d.head_dim // d.n_groups
    out = np.empty((d.batch, d.n_q_heads, d.n_groups, d.n_residuals, d.n_codes, W), dtype=np.float64)
    lib().oracle_table(ctypes.byref(d), _ptr(qq), _ptr(kb), _ptr(out))
    return out


def scores_via_table(d: Dims, tab, k_codes, seq_start, seq_len, max_len: int) -> np.ndarray:
    tt, kc = _f64(tab), _u8(k_codes)
    ss = np.ascontiguousarray(seq_start, dtype=np.int64)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    out = np.empty((d.batch, d.n_q_heads, max_len), dtype=np.float64)
    lib().oracle_scores_via_table(ctypes.byref(d), _ptr(tt), _ptr(kc), _ptr(ss), _ptr(sl), kc.shape[2], int(max_len),
                                  _ptr(out))
    return out


def value_reduce(d: Dims, p, v_codes, v_cb, seq_start, seq_len, max_len: int) -> np.ndarray:
    pp, vc, vb = _f64(p), _u8(v_codes), _f64(v_cb)
    assert pp.shape == (d.batch, d.n_q_heads, max_len)
    ss = np.ascontiguousarray(seq_start, dtype=np.int64)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    out = np.empty((d.batch, d.n_q_heads, d.head_dim), dtype=np.float64)
    lib().oracle_value_reduce(ctypes.byref(d), _ptr(pp), _ptr(vc), _ptr(vb), _ptr(ss), _ptr(sl), vc.shape[2],
                              int(max_len), _ptr(out))
    return out


def encode_greedy(d: Dims, x, codebook, want_dist: bool = False):
    """x [Hkv][n][D] in the codebook frame. Returns codes [Hkv][R][n][G] uint8 (and min distances)."""
    xx, cb = _f64(x), _f64(codebook)
    n = xx.shape[1]
    codes = np.empty((d.n_kv_heads, d.n_residuals, n, d.n_groups), dtype=np.uint8)
    dist = np.empty(codes.shape, dtype=np.float64) if want_dist else None
    lib().oracle_encode_greedy(ctypes.byref(d), _ptr(xx), _ptr(cb), int(n), _ptr(codes),
                               _ptr(dist) if dist is not None else None)
    return (codes, dist) if want_dist else codes


def encode_eval(d: Dims, x, codebook, codes):
    """Replay the greedy residual rounds with the given codes [Hkv][R][n][G]; returns (chosen, best, second)
    squared distances per round, each [Hkv][R][n][G] float64."""
    xx, cb, cc = _f64(x), _f64(codebook), _u8(codes)
    n = xx.shape[1]
    assert cc.shape == (d.n_kv_heads, d.n_residuals, n, d.n_groups)
    outs = [np.empty(cc.shape, dtype=np.float64) for _ in range(3)]
    lib().oracle_encode_eval(ctypes.byref(d), _ptr(xx), _ptr(cb), int(n), _ptr(cc), *(_ptr(o) for o in outs))
    return tuple(outs)


def codebook_update(d: Dims, x, codebook, codes, want_counts: bool = False):
    """One M-step of the residual codebook fit: x [Hkv][n][D], codebook [Hkv][G][R][N][W], codes
    [Hkv][R][n][G]. Returns the new codebook (float64, same shape) and optionally the per-codeword token
    counts [Hkv][G][R][N]."""
    xx, cb, cc = _f64(x), _f64(codebook), _u8(codes)
    n = xx.shape[1]
    assert cc.shape == (d.n_kv_heads, d.n_residuals, n, d.n_groups)
    out = np.empty(cb.shape, dtype=np.float64)
    counts = np.empty((d.n_kv_heads, d.n_groups, d.n_residuals, d.n_codes), dtype=np.int64) if want_counts else None
    lib().oracle_codebook_update(ctypes.byref(d), _ptr(xx), _ptr(cb), _ptr(cc), int(n), _ptr(out),
                                 _ptr(counts) if counts is not None else None)
    return (out, counts) if want_counts else out


def run_config(cfg, inputs, n_threads: int = 1):
    """Oracle output for a workloads config and its inputs dict (bit-packed records are unpacked here)."""
    d = dims_of(cfg)
    kc, vc = inputs["k_codes"], inputs["v_codes"]
    if kc.dtype == np.uint32:
        T = int(inputs["total_tokens"])
        kc, vc = unpack_bits(d, kc, T), unpack_bits(d, vc, T)
    return attn_decode(d, inputs["q"], kc, vc, inputs["k_cb"], inputs["v_cb"], inputs["seq_start"],
                       inputs["seq_len"], int(inputs["max_len"]), n_threads=n_threads)
