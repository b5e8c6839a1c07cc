"""Seeded synthetic inputs for CommVQ decode-step attention.

This module only draws random numbers and lays them out; it holds none of the method's arithmetic.
Both the HIP path's tests/benchmark and the CPU oracle read the same arrays from here.

Layouts (shared by every consumer):
  q        [B][Hq][D]              post-RoPE query, dtype = cfg.dtype (float16 or float32)
  k_cb     [Hkv][G][R][N][W]       key codebook: per RoPE pair of the group the block numbers (a, b)
  v_cb     [Hkv][G][R][N][W]       value codebook
  k_codes  [Hkv][R][T][G] uint8    one byte per code index (N = 256); one plane per residual
  v_codes  [Hkv][R][T][G] uint8
           N < 256 (the pages' g = 64 setting, N = 64): bit-packed word planes [Hkv][words][T] uint32
           instead: each token's R*G indices of log2(N) bits as one little-endian bitstream, index (r, g) at
           bit log2(N) * (r*G + g), words = ceil(log2(N) * R * G / 32), word w of token t at [kv][w][t]
  seq_start[B] int64, seq_len[B] int32: sequence b owns token rows seq_start[b] .. +seq_len[b]-1
with D = head_dim, G = n_groups, W = D / G, R = n_residuals, N = n_codes, T = total tokens.

Distributions: codebook entries N(0, variance 0.25) drawn in float32 then rounded to the storage
dtype (round to nearest even); q ~ N(0, q_std^2) likewise (q_std = 1 unless a config widens the logit
range); code indices uniform on [0, N). Draw order per seed: lengths (ragged only), k_cb, v_cb, q,
k_codes, v_codes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    lengths: Optional[tuple]  # fixed per-sequence lengths, or None for ragged draws
    n_residuals: int
    dtype: str  # "float16" | "float32"
    seed: int
    head_dim: int = 128
    n_groups: int = 16
    n_codes: int = 256
    rope_base: float = 500000.0
    ragged_range: Optional[tuple] = None  # (lo, hi) inclusive for ragged lengths
    q_std: float = 1.0  # standard deviation of the query entries (wider logit ranges for larger values)
    description: str = ""

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group_dim(self) -> int:
        return self.head_dim // self.n_groups

    @property
    def index_bits(self) -> int:
        return int(round(math.log2(self.n_codes)))

    @property
    def packed(self) -> bool:
        """Bit-packed token records (N < 256) instead of one byte per index."""
        return self.n_codes < 256

    @property
    def record_words(self) -> int:
        return (self.index_bits * self.n_residuals * self.n_groups + 31) // 32


# The five workloads: a tiny CPU-checkable step, the Llama-3.1-8B layer shape (8 KV / 32 q heads,
# head dim 128) at 8K / 32K / 128K context, and a ragged batch of 16 sequences.
CONFIGS: Dict[str, Config] = {
    "tiny_1k_r2_f32": Config("tiny_1k_r2_f32", 1, 4, 1, (1024,), 2, "float32", 0,
                             description="B=1, 1 KV head, 4 q heads, L=1024, 2-bit (R=2), fp32"),
    "llama8b_8k_r2": Config("llama8b_8k_r2", 1, 32, 8, (8192,), 2, "float16", 1,
                            description="Llama-3.1-8B layer, L=8192, 2-bit (R=2), fp16"),
    "llama8b_32k_r1": Config("llama8b_32k_r1", 1, 32, 8, (32768,), 1, "float16", 2,
                             description="Llama-3.1-8B layer, L=32768, 1-bit (R=1), fp16"),
    "llama8b_128k_r1": Config("llama8b_128k_r1", 1, 32, 8, (131072,), 1, "float16", 3,
                              description="Llama-3.1-8B layer, L=131072, 1-bit (R=1), fp16"),
    "llama8b_128k_r2": Config("llama8b_128k_r2", 1, 32, 8, (131072,), 2, "float16", 4,
                              description="Llama-3.1-8B layer, L=131072, 2-bit (R=2), fp16"),
    "ragged16_r2": Config("ragged16_r2", 16, 32, 8, None, 2, "float16", 5, ragged_range=(4096, 65536),
                          description="16 sequences, L_b ~ U[4096, 65536], 2-bit (R=2), fp16"),
}

# The pages' own setting: one index shared by 64 dims (G = 2 groups of 64), N' = 64 codewords (6-bit
# indices, bit-packed), R = 11 (1.03 bits per scalar) or R = 21 (1.97 bits), at the same layer shape.
PAGES_CONFIGS: Dict[str, Config] = {
    "pages_g64_r11_small": Config("pages_g64_r11_small", 2, 8, 2, (1000, 3001), 11, "float16", 20, n_groups=2,
                                  n_codes=64, description="g=64, N'=64, R=11, two short sequences, fp16"),
    "pages_g64_r11_32k": Config("pages_g64_r11_32k", 1, 32, 8, (32768,), 11, "float16", 21, n_groups=2, n_codes=64,
                                description="Llama-3.1-8B layer, L=32768, g=64, N'=64, R=11 (1.03 bit), fp16"),
    "pages_g64_r21_32k": Config("pages_g64_r21_32k", 1, 32, 8, (32768,), 21, "float16", 22, n_groups=2, n_codes=64,
                                description="Llama-3.1-8B layer, L=32768, g=64, N'=64, R=21 (1.97 bit), fp16"),
    "pages_g64_r21_128k": Config("pages_g64_r21_128k", 1, 32, 8, (131072,), 21, "float16", 23, n_groups=2,
                                 n_codes=64, description="Llama-3.1-8B layer, L=131072, g=64, N'=64, R=21, fp16"),
    "pages_g64_r11_128k": Config("pages_g64_r11_128k", 1, 32, 8, (131072,), 11, "float16", 24, n_groups=2,
                                 n_codes=64, description="Llama-3.1-8B layer, L=131072, g=64, N'=64, R=11, fp16"),
}


def custom(name: str, batch: int, n_q_heads: int, n_kv_heads: int, lengths, n_residuals: int, dtype: str,
           seed: int, **kw) -> Config:
    """A config of arbitrary shape (tests use this for small, ragged and edge cases)."""
    return Config(name, batch, n_q_heads, n_kv_heads, tuple(int(x) for x in lengths), n_residuals, dtype, seed, **kw)


def draw_lengths(cfg: Config, rng: np.random.Generator) -> List[int]:
    if cfg.lengths is not None:
        assert len(cfg.lengths) == cfg.batch
        return list(cfg.lengths)
    lo, hi = cfg.ragged_range
    return [int(x) for x in rng.integers(lo, hi + 1, size=cfg.batch)]


def make_inputs(cfg: Config, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Deterministic inputs for `cfg` (seed defaults to cfg.seed). Returns numpy arrays."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    dt = np.dtype(cfg.dtype)
    lengths = draw_lengths(cfg, rng)
    B, Hq, Hkv, D = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G, R, N, W = cfg.n_groups, cfg.n_residuals, cfg.n_codes, cfg.group_dim
    seq_len = np.asarray(lengths, dtype=np.int32)
    seq_start = np.zeros(B, dtype=np.int64)
    if B > 1:
        seq_start[1:] = np.cumsum(seq_len[:-1], dtype=np.int64)
    total = int(seq_len.sum())
    k_cb = (rng.standard_normal((Hkv, G, R, N, W), dtype=np.float32) * np.float32(0.5)).astype(dt)
    v_cb = (rng.standard_normal((Hkv, G, R, N, W), dtype=np.float32) * np.float32(0.5)).astype(dt)
    q = (rng.standard_normal((B, Hq, D), dtype=np.float32) * np.float32(cfg.q_std)).astype(dt)
    k_codes = rng.integers(0, N, size=(Hkv, R, total, G), dtype=np.uint8) if N == 256 else \
        rng.integers(0, N, size=(Hkv, R, total, G)).astype(np.uint8)
    v_codes = rng.integers(0, N, size=(Hkv, R, total, G), dtype=np.uint8) if N == 256 else \
        rng.integers(0, N, size=(Hkv, R, total, G)).astype(np.uint8)
    if cfg.packed:
        k_codes, v_codes = pack_bits(k_codes, cfg.index_bits), pack_bits(v_codes, cfg.index_bits)
    return dict(q=q, k_cb=k_cb, v_cb=v_cb, k_codes=k_codes, v_codes=v_codes, seq_start=seq_start,
                seq_len=seq_len, total_tokens=np.int64(total), max_len=np.int32(max(lengths) if lengths else 0))


def pack_bits(idx: np.ndarray, bits: int) -> np.ndarray:
    """Lay out indices [Hkv][R][T][G] (each < 2**bits) as bit-packed word planes [Hkv][words][T] uint32."""
    Hkv, R, T, G = idx.shape
    words = (bits * R * G + 31) // 32
    out = np.zeros((Hkv, words, T), dtype=np.uint64)
    for r in range(R):
        for g in range(G):
            pos = bits * (r * G + g)
            w, sh = pos // 32, pos % 32
            v = idx[:, r, :, g].astype(np.uint64)
            out[:, w, :] |= (v << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
            if sh + bits > 32:
                out[:, w + 1, :] |= v >> np.uint64(32 - sh)
    return out.astype(np.uint32)


def code_bytes(cfg: Config, total_tokens: int) -> int:
    """Bytes of key + value code indices for `total_tokens` cached tokens (all KV heads)."""
    if cfg.packed:
        return 2 * cfg.n_kv_heads * total_tokens * cfg.record_words * 4
    return 2 * cfg.n_kv_heads * total_tokens * cfg.n_residuals * cfg.n_groups
