"""Seeded synthetic inputs for the quantized-KV decode path.

This module only draws random data and rounds it to 16-bit storage; it holds
none of the quantization, selection or attention arithmetic.  The GPU library
(through its Python binding) and the CPU oracle both consume its output as
plain data (16-bit bit patterns in numpy ``uint16`` arrays).

Recipe (the pages publish no data; every workload here is synthetic):
  * ``numpy.random.default_rng(seed)`` (PCG64), fp64 N(0, 1) draws in the
    order: selection queries, keys (prefill + appended tokens), values
    (prefill + appended), decode queries, then the outlier picks.
  * Outlier key pairs, per the workload: ``"pairs4x8"`` picks 4 distinct RoPE
    pairs per (sequence, KV head) and scales both of their channels x8 at
    every position; ``"pct2x10"`` picks round(0.02 * Hkv * 64) distinct
    (KV head, pair) slots per sequence and scales them x10.
  * RoPE (rotate-half pairing: pair j = channels j and j+64, base 1e4) is
    applied in fp64 to keys at positions 0.., to the selection queries at the
    last ``n_qry`` prefill positions and to decode query i at position T + i.
    The quantization library receives post-RoPE vectors; RoPE itself is part
    of the model, not of the library.
  * Rounding to the I/O dtype: fp16 by numpy's RNE cast; bf16 by RNE from the
    value first rounded to fp32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 128
N_PAIRS = 64
ROPE_BASE = 1.0e4


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, bit allocation and data recipe of one synthetic workload."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    tokens: int              # prefill tokens T
    n_qry: int = 64          # selection queries per query head
    n_dec: int = 1           # decode queries (one per decode step)
    n_app: int = 0           # appended tokens (streaming decode)
    io_dtype: str = "bf16"   # "fp16" | "bf16"
    outliers: str = "pairs4x8"
    n_pairs_hi: int = 6
    bits_hi: int = 4
    n_pairs_lo1: int = 0     # lowest-ranked pairs kept at 1 bit
    residual: int = 128
    n_splits: int = 0        # 0 = library default
    seed: int = 0
    n_vblk_hi: int = 0       # per group, 8 * n_vblk_hi tokens (largest keys) get bits_vhi-bit values
    bits_vhi: int = 4
    prog_w8: int = 0         # progressive precision: newest groups held at 8 bits
    prog_w4: int = 0         # ... and at 4 bits or more (0: off)

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_tokens(self) -> int:
        return self.tokens + self.n_app

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, seed = 1000 + index, and one measurement variant.
WORKLOADS = [
    Workload("tiny", 1, 1, 1, 512, io_dtype="fp16", outliers="pairs4x8",
             n_pairs_hi=8, residual=32, seed=1000),
    Workload("llama3-8b-32k", 1, 32, 8, 32768, outliers="pct2x10",
             n_pairs_hi=6, residual=128, seed=1001),
    Workload("streaming-b16", 16, 32, 8, 4096, n_dec=512, n_app=512,
             outliers="pairs4x8", n_pairs_hi=6, residual=128, seed=1002),
    Workload("pareto-b4-16k", 4, 32, 8, 16384, outliers="pct2x10",
             n_pairs_hi=6, residual=128, seed=1003),
    # 256 token partitions in all: 32 per KV head, one workgroup per CU
    Workload("long-128k", 1, 64, 8, 131072, outliers="pairs4x8",
             n_pairs_hi=6, residual=128, n_splits=32, seed=1004),
    # the 32K layer's cache with one query head per KV head (G = 1): the same
    # bytes, 1 of 16 MFMA head columns used
    # progressive precision: 256 quantized groups (8192 tokens) plus the
    # residual, so that the widest windows hold every group
    Workload("prog-8k", 1, 32, 8, 8192 + 128, outliers="pct2x10",
             n_pairs_hi=6, residual=128, seed=1006),
    Workload("prog-32k", 1, 32, 8, 32768, outliers="pct2x10",
             n_pairs_hi=6, residual=128, seed=1007),
    Workload("g1-32k", 1, 8, 8, 32768, outliers="pct2x10",
             n_pairs_hi=6, residual=128, seed=1005),
]

# Key bit points of the Pareto sweep: (label, n_pairs_hi, bits_hi).
# Bit points of the precision sweep: (label, salient pairs, their bits,
# pairs at 1 bit).  "1.5": 32 pairs at 2 bits and the 32 lowest-ranked at 1.
PARETO_POINTS = [("1.5", 0, 4, 32), ("2.0", 0, 4, 0), ("2.26", 6, 4, 0), ("3.0", 6, 16, 0)]
# Value-precision points on the 2.26-bit keys: (label, kept 8-token value
# blocks per 32-token group, their bits).
VALUE_POINTS = [("2.26 v1@3", 1, 3), ("2.26 v1@4", 1, 4), ("2.26 v2@4", 2, 4)]
# Progressive-precision windows (label, groups held at 8 bits, groups held
# at 4 bits or more): the plain cache, a steady state, every group at 4 bits,
# every group at 8 bits (up to 256 groups: the cache before any shrink).
PROG_POINTS = [("2-bit", 0, 0), ("8/4/2 windows 4/16", 4, 16), ("4-bit, 256 groups", 0, 256),
               ("8-bit, 256 groups", 256, 256)]


def workload(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def _rope(x: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE in fp64 along the last axis; ``pos`` broadcasts over
    the token axis (second to last)."""
    j = np.arange(N_PAIRS, dtype=np.float64)
    theta = ROPE_BASE ** (-2.0 * j / HEAD_DIM)
    ang = pos.astype(np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :N_PAIRS], x[..., N_PAIRS:]
    out = np.empty_like(x)
    out[..., :N_PAIRS] = a * c - b * s
    out[..., N_PAIRS:] = a * s + b * c
    return out


def to_bits(x: np.ndarray, io_dtype: str) -> np.ndarray:
    """Round fp64 data to the 16-bit I/O dtype; returns the bit patterns."""
    if io_dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if io_dtype == "bf16":
        u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
        return r
    raise ValueError(io_dtype)


def _outlier_scale(rng, w: Workload) -> np.ndarray:
    """Per-(b, kv head, pair) key multiplier."""
    m = np.ones((w.batch, w.n_kv_heads, N_PAIRS))
    if w.outliers == "pairs4x8":
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                m[b, h, rng.choice(N_PAIRS, 4, replace=False)] = 8.0
    elif w.outliers == "pct2x10":
        n = int(round(0.02 * w.n_kv_heads * N_PAIRS))
        for b in range(w.batch):
            flat = m[b].reshape(-1)
            flat[rng.choice(w.n_kv_heads * N_PAIRS, n, replace=False)] = 10.0
    elif w.outliers != "none":
        raise ValueError(w.outliers)
    return m


def generate(w: Workload, keep_pre_rope: bool = False) -> dict:
    """Draw the workload's inputs.

    Returns a dict of uint16 bit arrays (``q_sel`` [B][Hq][n_qry][128],
    ``k``/``v`` [B][Hkv][T + n_app][128], ``q_dec`` [B][Hq][n_dec][128]) plus
    ``outlier_scale`` [B][Hkv][64].  With ``keep_pre_rope`` it also returns
    the fp64 arrays before and after RoPE (``*_pre``/``*_post``) for checks
    of the RoPE step.
    """
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, T = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens
    Tt = T + w.n_app
    q_sel = rng.standard_normal((B, Hq, w.n_qry, HEAD_DIM))
    k = rng.standard_normal((B, Hkv, Tt, HEAD_DIM))
    v = rng.standard_normal((B, Hkv, Tt, HEAD_DIM))
    q_dec = rng.standard_normal((B, Hq, w.n_dec, HEAD_DIM))
    scale = _outlier_scale(rng, w)
    k *= np.concatenate([scale, scale], axis=-1)[:, :, None, :]

    out = {"outlier_scale": scale}
    if keep_pre_rope:
        out.update(q_sel_pre=q_sel.copy(), k_pre=k.copy(), q_dec_pre=q_dec.copy())
    q_sel = _rope(q_sel, np.arange(T - w.n_qry, T))
    k = _rope(k, np.arange(Tt))
    q_dec = _rope(q_dec, np.arange(T, T + w.n_dec))
    if keep_pre_rope:
        out.update(q_sel_post=q_sel, k_post=k, q_dec_post=q_dec)
    out["q_sel"] = to_bits(q_sel, w.io_dtype)
    out["k"] = to_bits(k, w.io_dtype)
    out["v"] = to_bits(v, w.io_dtype)
    out["q_dec"] = to_bits(q_dec, w.io_dtype)
    return out


def bits_to_f64(bits: np.ndarray, io_dtype: str) -> np.ndarray:
    """Widen 16-bit patterns to fp64 with numpy's own casts (data plumbing)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if io_dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
