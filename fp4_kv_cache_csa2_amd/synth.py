"""Seeded synthetic inputs for the CSA2 global-branch hot path.

This module only draws random numbers and lays them out in the shapes the path consumes.
It holds none of the method's arithmetic (no pooling, rotation, quantisation, scoring,
selection or attention) and imports neither the HIP binding nor the oracle: both the
GPU tests and the oracle consume the arrays it returns.

Recipe (numpy ``Generator(PCG64(seed))``, draws in this order):
  latents      N(0,1) per channel, each 512-row divided by sqrt(mean(x^2) + 1e-6), -> bf16
  pool weights softplus(N(0,1)) per (i, channel), fp32 [m, 512]
  W_idx        N(0,1) / sqrt(512) -> bf16 [128, 512]
  q_idx        N(0,1) / sqrt(128) -> bf16 [n_q, 32, 128]  (``q_idx_scale`` overrides)
  head_w       N(0,1) / sqrt(32)  fp32 [n_q, 32]
  main q       N(0,1) -> bf16 [n_q, 64, 512]; a rotation of an isotropic Gaussian pair
               is the same Gaussian, so drawing the post-RoPE query directly has the
               distribution of RoPE applied to N(0,1)
  SWA rows     drawn like the latents, bf16 [rows, 512]
Entry j of a ratio-m layer takes its RoPE angle at token position m*j.

For the full-size decode workloads the packed caches themselves are drawn directly
(uniform E2M1 nibbles, scale bytes from a narrow realistic band): see ``random_caches``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_LAT = 512
N_HEADS = 64
IDX_HEADS = 32
IDX_DIM = 128
KV_BYTES = 288
IDX_BYTES = 68
ROPE_THETA = 160000.0


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rms_rows(rng: np.random.Generator, rows: int) -> np.ndarray:
    x = rng.standard_normal((rows, D_LAT), dtype=np.float32)
    x /= np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True) + 1e-6).astype(np.float32)
    return f32_to_bf16_bits(x)


def softplus_weights(rng: np.random.Generator, m: int) -> np.ndarray:
    z = rng.standard_normal((m, D_LAT)).astype(np.float64)
    return np.log1p(np.exp(z)).astype(np.float32)


@dataclass
class CompressInputs:
    latent: np.ndarray  # uint16 [n*m, 512]
    m: int
    pool_w: np.ndarray  # fp32 [m, 512]
    w_idx: np.ndarray  # uint16 [128, 512]
    positions: np.ndarray  # int64 [n] token position of each entry


def compress_inputs(seed: int, n_entries: int, m: int, first_entry: int = 0) -> CompressInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    latent = rms_rows(rng, n_entries * m)
    pool_w = softplus_weights(rng, m)
    w_idx = f32_to_bf16_bits(rng.standard_normal((IDX_DIM, D_LAT), dtype=np.float32) / np.sqrt(512.0))
    pos = (np.arange(n_entries, dtype=np.int64) + first_entry) * m
    return CompressInputs(latent, m, pool_w, w_idx, pos)


@dataclass
class DecodeInputs:
    q_idx: np.ndarray  # uint16 [n_q, 32, 128]
    head_w: np.ndarray  # fp32 [n_q, 32]
    q: np.ndarray  # uint16 [n_q, 64, 512]
    swa: np.ndarray  # uint16 [rows, 512]
    swa_start: np.ndarray  # int64 [n_q]
    swa_len: np.ndarray  # int32 [n_q]


def query_inputs(seed: int, n_q: int, q_idx_scale: float | None = None,
                 swa_rows: int | None = None, swa_start=None, swa_len=None) -> DecodeInputs:
    """Indexer query, head weights, main query and SWA rows for n_q queries.

    By default every query owns 128 window rows (rows 128 t .. 128 t + 127)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = (1.0 / np.sqrt(128.0)) if q_idx_scale is None else q_idx_scale
    q_idx = f32_to_bf16_bits(rng.standard_normal((n_q, IDX_HEADS, IDX_DIM), dtype=np.float32) * np.float32(s))
    head_w = (rng.standard_normal((n_q, IDX_HEADS), dtype=np.float32) / np.float32(np.sqrt(32.0))).astype(np.float32)
    q = f32_to_bf16_bits(rng.standard_normal((n_q, N_HEADS, D_LAT), dtype=np.float32))
    if swa_rows is None:
        swa_rows = 128 * n_q
    swa = rms_rows(rng, swa_rows)
    if swa_start is None:
        swa_start = np.arange(n_q, dtype=np.int64) * 128
    if swa_len is None:
        swa_len = np.full(n_q, 128, np.int32)
    return DecodeInputs(q_idx, head_w, q, swa, np.asarray(swa_start, np.int64), np.asarray(swa_len, np.int32))


def random_caches(seed: int, n_entries: int, spread_scales: bool = False):
    """Directly drawn packed caches with the entry structure of the pages' formats.

    Main KV: 256 uniform payload bytes + 32 E4M3 scale bytes uniform in [0x20, 0x38]
    (scales 0.125 .. 1.0).  Indexer K: 64 uniform payload bytes + 4 E8M0 scale bytes
    uniform in [124, 127] (2^-3 .. 2^0).

    spread_scales: the scale bytes cover every non-negative finite E4M3 code (0x00 .. 0x7E:
    0, the subnormals 2^-9 .. and up to 448) and the E8M0 codes 16 .. 240 (2^-111 .. 2^113:
    the widest band whose scores stay finite in fp32 with this module's query scale)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = np.empty((n_entries, KV_BYTES), np.uint8)
    kv[:, :256] = rng.integers(0, 256, (n_entries, 256), dtype=np.uint8)
    lo, hi = (0x00, 0x7F) if spread_scales else (0x20, 0x39)
    kv[:, 256:] = rng.integers(lo, hi, (n_entries, 32), dtype=np.uint8)
    ix = np.empty((n_entries, IDX_BYTES), np.uint8)
    ix[:, :64] = rng.integers(0, 256, (n_entries, 64), dtype=np.uint8)
    lo, hi = (16, 241) if spread_scales else (124, 128)
    ix[:, 64:] = rng.integers(lo, hi, (n_entries, 4), dtype=np.uint8)
    return kv, ix


def random_scores(seed: int, n_q: int, width: int, tie_frac: float = 0.0, levels: int = 0,
                  nan_frac: float = 0.0) -> np.ndarray:
    """fp32 score rows for selection tests.

    tie_frac: fraction of positions overwritten with a copy of another position's score.
    levels:   if > 0, scores are quantised to that many distinct values (massive ties).
    nan_frac: fraction of positions set to NaN."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = rng.standard_normal((n_q, width)).astype(np.float32)
    if levels > 0:
        s = np.floor(s * levels / 4.0).astype(np.float32)
    if tie_frac > 0:
        k = int(tie_frac * width)
        for t in range(n_q):
            dst = rng.integers(0, width, k)
            src = rng.integers(0, width, k)
            s[t, dst] = s[t, src]
    if nan_frac > 0:
        mask = rng.random((n_q, width)) < nan_frac
        s[mask] = np.nan
    return s


# ------------------------------------------------------------------ workloads
@dataclass
class Workload:
    """One of the seeded synthetic configurations (sizes only; arrays are drawn lazily)."""
    name: str
    seed: int
    m: int
    n_seq: int
    tokens: int  # tokens per sequence (entries = tokens // m)
    n_q: int  # decode queries (one per sequence) or prefill chunk queries
    desc: str = ""
    layers: tuple = ("full",)
    prefill_chunk: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def entries(self) -> int:
        return self.tokens // self.m


WORKLOADS = {
    "tiny_decode_m2": Workload(
        "tiny_decode_m2", 0, 2, 1, 4096, 1,
        "1 sequence, 4096 tokens -> 2048 entries, 256 blocks (pool covers all), 1 query"),
    "decode_m1_b4_32k": Workload(
        "decode_m1_b4_32k", 1, 1, 4, 32768, 4,
        "batch 4 decode over 32768 entries each, 4096 blocks -> 2048 -> Top-512"),
    "decode_128k_b16_full_reindex_reuse": Workload(
        "decode_128k_b16_full_reindex_reuse", 2, 1, 16, 131072, 16,
        "batch 16 decode, 128K entries: Full + Reindex (pool 2048x8) + 3 Reuse layers",
        layers=("full", "reindex", "reuse", "reuse", "reuse")),
    "decode_1m_b4_m2": Workload(
        "decode_1m_b4_m2", 3, 2, 4, 1048576, 4,
        "batch 4 decode, 1M tokens -> 524288 FP4 entries per sequence, Full layer"),
    "prefill_chunk4096_hist65536_m2": Workload(
        "prefill_chunk4096_hist65536_m2", 4, 2, 1, 65536 + 4096, 4096,
        "4096-query chunk on a 65536-token history at m=2: compress 2048 new entries, "
        "causal indexer 4096 x <=34816, per-query Top-512, sparse attention",
        prefill_chunk=4096),
}


def prefill_nvis(hist_tokens: int, chunk: int, m: int) -> np.ndarray:
    """Visible complete entries for chunk query i at token hist_tokens + i: floor((t+1)/m)."""
    t = hist_tokens + np.arange(chunk, dtype=np.int64)
    return ((t + 1) // m).astype(np.int32)
