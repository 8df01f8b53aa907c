"""Plain CPU oracle for the CSA2 global-branch hot path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path (the
HIP library and its Python binding) never imports, links or calls anything here, and
this package imports nothing from the product path.

The arithmetic lives in ``csa2_oracle.c`` (plain single-threaded C, ``-O2
-ffp-contract=off``); this module only builds it with gcc and marshals numpy arrays.
Every function cites the passage of the pages it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "libcsa2_oracle.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared", "-Wall"]

KV_BYTES = 288
IDX_BYTES = 68
D_LAT = 512
N_HEADS = 64
IDX_HEADS = 32
IDX_DIM = 128


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/libcsa2_oracle.so`` with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        i32, i64, f64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.csa2o_entry_bytes.argtypes = [i64, i64]
        L.csa2o_entry_bytes.restype = i64
        L.csa2o_e2m1_value.argtypes = [ctypes.c_int]
        L.csa2o_e2m1_value.restype = f64
        L.csa2o_e4m3_value.argtypes = [ctypes.c_int]
        L.csa2o_e4m3_value.restype = f64
        L.csa2o_e8m0_value.argtypes = [ctypes.c_int]
        L.csa2o_e8m0_value.restype = f64
        L.csa2o_e4m3_encode.argtypes = [f64]
        L.csa2o_e4m3_encode.restype = ctypes.c_int
        L.csa2o_e2m1_encode.argtypes = [ctypes.c_float, f64]
        L.csa2o_e2m1_encode.restype = ctypes.c_int
        L.csa2o_e8m0_scale_code.argtypes = [ctypes.c_float]
        L.csa2o_e8m0_scale_code.restype = ctypes.c_int
        L.csa2o_rope_table.argtypes = [vp, i64, f64, vp]
        L.csa2o_compress_pack.argtypes = [vp, i64, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
        L.csa2o_dequant_kv.argtypes = [vp, vp]
        L.csa2o_dequant_idx.argtypes = [vp, vp]
        L.csa2o_index_score.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
        L.csa2o_block_topk.argtypes = [vp, i32, i32, vp, vp, i32, i32, i32, vp, vp]
        L.csa2o_topk_bruteforce.argtypes = [vp, i32, i32, vp, i32, vp]
        L.csa2o_sparse_attn.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, ctypes.c_float, vp, vp, i32]
        L.csa2o_quantize_q_mxfp4.argtypes = [vp, i64, vp]
        L.csa2o_index_score_fp4q.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
        L.csa2o_block_mean_pack.argtypes = [vp, i64, i32, vp]
        L.csa2o_pool_from_block_scores.argtypes = [vp, i32, i32, vp, i32, i32, vp]
        L.csa2o_swa_fp8_row_bytes.argtypes = []
        L.csa2o_swa_fp8_row_bytes.restype = i64
        L.csa2o_e8m0_scale_code_e4m3.argtypes = [ctypes.c_float]
        L.csa2o_e8m0_scale_code_e4m3.restype = ctypes.c_int
        L.csa2o_swa_fp8_pack.argtypes = [vp, i64, vp]
        L.csa2o_dequant_swa_fp8.argtypes = [vp, vp]
        L.csa2o_sparse_attn_swa_fp8.argtypes = [vp, vp, vp, vp, i32, vp, i64, vp, vp, ctypes.c_float, vp, vp, i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalar formats
def entry_bytes(D: int, G: int) -> int:
    return int(lib().csa2o_entry_bytes(D, G))


def e2m1_value(code: int) -> float:
    return lib().csa2o_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    return lib().csa2o_e4m3_value(byte)


def e8m0_value(byte: int) -> float:
    return lib().csa2o_e8m0_value(byte)


def e4m3_encode(x: float) -> int:
    return lib().csa2o_e4m3_encode(float(x))


def e2m1_encode(e: float, S: float) -> int:
    return lib().csa2o_e2m1_encode(float(e), float(S))


def e8m0_scale_code(amax: float) -> int:
    return lib().csa2o_e8m0_scale_code(float(amax))


# ---------------------------------------------------------------- table
def rope_table(pos, theta: float = 160000.0) -> np.ndarray:
    pos = _c(pos, np.int64)
    out = np.empty((pos.size, 64), np.float32)
    lib().csa2o_rope_table(_p(pos), pos.size, float(theta), _p(out))
    return out


# ---------------------------------------------------------------- stage 1
def compress_pack(latent_bf16, m: int, pool_w, rope_cs, w_idx_bf16, intermediates: bool = False):
    """latent_bf16 uint16 [n*m, 512] -> (kv uint8 [n, 288], idx uint8 [n, 68][, pooled, rotated, k]).

    pool_w is fp32 [m, 512] (static per-channel weights) or [n*m, 512] (one weight row per
    latent token: per-token gates, same formula)."""
    latent = _c(latent_bf16, np.uint16)
    n = latent.shape[0] // m
    pw = None if pool_w is None else _c(pool_w, np.float32)
    per_token = pw is not None and m > 1 and pw.shape[0] == n * m and n * m != m
    assert pw is None or pw.shape[0] in (m, n * m)
    cs = _c(rope_cs, np.float32)
    w = _c(w_idx_bf16, np.uint16)
    assert cs.shape == (n, 64) and w.shape == (128, 512)
    kv = np.empty((n, KV_BYTES), np.uint8)
    ix = np.empty((n, IDX_BYTES), np.uint8)
    pooled = rotated = kproj = None
    if intermediates:
        pooled = np.empty((n, D_LAT), np.float32)
        rotated = np.empty((n, D_LAT), np.float32)
        kproj = np.empty((n, IDX_DIM), np.float32)
    lib().csa2o_compress_pack(_p(latent), n, m, _p(pw), int(per_token), _p(cs), _p(w), _p(kv), _p(ix),
                              _p(pooled), _p(rotated), _p(kproj))
    if intermediates:
        return kv, ix, pooled, rotated, kproj
    return kv, ix


def dequant_kv(entries) -> np.ndarray:
    e = _c(entries, np.uint8).reshape(-1, KV_BYTES)
    out = np.empty((e.shape[0], D_LAT), np.float64)
    for i in range(e.shape[0]):
        lib().csa2o_dequant_kv(_p(e[i]), _p(out[i]))
    return out


def dequant_idx(entries) -> np.ndarray:
    e = _c(entries, np.uint8).reshape(-1, IDX_BYTES)
    out = np.empty((e.shape[0], IDX_DIM), np.float64)
    for i in range(e.shape[0]):
        lib().csa2o_dequant_idx(_p(e[i]), _p(out[i]))
    return out


# ---------------------------------------------------------------- stage 2
def index_score(q_idx_bf16, head_w, idx_cache, q_base, q_nvis, width: int,
                pool_blocks=None, M: int = 0) -> np.ndarray:
    q = _c(q_idx_bf16, np.uint16)
    w = _c(head_w, np.float32)
    cache = _c(idx_cache, np.uint8)
    base = _c(q_base, np.int64)
    nvis = _c(q_nvis, np.int32)
    n_q = base.size
    pb = None
    if pool_blocks is not None:
        pb = _c(pool_blocks, np.int32)
        M = pb.shape[1]
    out = np.empty((n_q, width), np.float32)
    lib().csa2o_index_score(_p(q), _p(w), _p(cache), _p(base), _p(nvis), _p(pb), M, n_q, width, _p(out))
    return out


def quantize_q_mxfp4(q_bf16):
    """Indexer query bf16 bits [n_q, 32, 128] -> MXFP4 head vectors uint8 [n_q, 32, 68]."""
    q = _c(q_bf16, np.uint16)
    n_q = q.shape[0]
    out = np.empty((n_q, IDX_HEADS, IDX_BYTES), np.uint8)
    lib().csa2o_quantize_q_mxfp4(_p(q), n_q * IDX_HEADS, _p(out))
    return out


def index_score_fp4q(q_fp4, head_w, idx_cache, q_base, q_nvis, width: int, pool_blocks=None, M: int = 0):
    q = _c(q_fp4, np.uint8)
    w = _c(head_w, np.float32)
    cache = _c(idx_cache, np.uint8)
    base = _c(q_base, np.int64)
    nvis = _c(q_nvis, np.int32)
    n_q = base.size
    pb = None
    if pool_blocks is not None:
        pb = _c(pool_blocks, np.int32)
        M = pb.shape[1]
    out = np.empty((n_q, width), np.float32)
    lib().csa2o_index_score_fp4q(_p(q), _p(w), _p(cache), _p(base), _p(nvis), _p(pb), M, n_q, width, _p(out))
    return out


def block_mean_pack(idx_cache, block: int = 8):
    """HISA block means of one sequence's indexer keys: uint8 [n, 68] -> [ceil(n/block), 68]."""
    cache = _c(idx_cache, np.uint8)
    n = cache.shape[0]
    out = np.empty(((n + block - 1) // block, IDX_BYTES), np.uint8)
    lib().csa2o_block_mean_pack(_p(cache), n, block, _p(out))
    return out


def pool_from_block_scores(block_scores, q_nvis, M: int = 2048, block: int = 8):
    """Top-M blocks of block_scores [n_q, nbw] (newest visible block forced), ascending, -1 pad."""
    bs = _c(block_scores, np.float32)
    nvis = _c(q_nvis, np.int32)
    n_q, nbw = bs.shape
    out = np.empty((n_q, M), np.int32)
    lib().csa2o_pool_from_block_scores(_p(bs), n_q, nbw, _p(nvis), block, M, _p(out))
    return out


# ---------------------------------------------------------------- stage 3
def block_topk(scores, q_nvis, K: int = 512, M: int = 2048, block: int = 8,
               pool_blocks=None, want_pool: bool = True):
    s = _c(scores, np.float32)
    n_q, width = s.shape
    nvis = _c(q_nvis, np.int32)
    pb = None
    if pool_blocks is not None:
        pb = _c(pool_blocks, np.int32)
        M = pb.shape[1]
    pool = np.empty((n_q, M), np.int32) if (pb is None and want_pool) else None
    topk = np.empty((n_q, K), np.int32)
    lib().csa2o_block_topk(_p(s), n_q, width, _p(nvis), _p(pb), block, M, K, _p(pool), _p(topk))
    return pool, topk


def topk_bruteforce(scores, q_nvis, K: int = 512) -> np.ndarray:
    s = _c(scores, np.float32)
    n_q, width = s.shape
    nvis = _c(q_nvis, np.int32)
    topk = np.empty((n_q, K), np.int32)
    lib().csa2o_topk_bruteforce(_p(s), n_q, width, _p(nvis), K, _p(topk))
    return topk


# ---------------------------------------------------------------- stage 4
def sparse_attn(q_bf16, kv_cache, q_base, topk, swa_bf16, swa_start, swa_len,
                scale: float = 1.0 / np.sqrt(512.0)):
    q = _c(q_bf16, np.uint16)
    n_q = q.shape[0]
    cache = _c(kv_cache, np.uint8)
    base = _c(q_base, np.int64)
    tk = _c(topk, np.int32)
    K = tk.shape[1]
    swa = _c(swa_bf16, np.uint16)
    ss = _c(swa_start, np.int64)
    sl = _c(swa_len, np.int32)
    out = np.empty((n_q, N_HEADS, D_LAT), np.float32)
    lse = np.empty((n_q, N_HEADS), np.float32)
    lib().csa2o_sparse_attn(_p(q), _p(cache), _p(base), _p(tk), K, _p(swa), _p(ss), _p(sl),
                            float(scale), _p(out), _p(lse), n_q)
    return out, lse


# ---- FP8 window rows: the sliding-window KV kept in FP8 ([ZB] §2.4.4; the 584-byte FP8 KV
# entry of [ZB] §3.1 and [DF] §4.6)
def swa_fp8_row_bytes() -> int:
    return int(lib().csa2o_swa_fp8_row_bytes())


def e8m0_scale_code_e4m3(amax: float) -> int:
    return int(lib().csa2o_e8m0_scale_code_e4m3(float(amax)))


def swa_fp8_pack(rows_bf16):
    """bf16 rows [n, 512] (uint16 bits) -> FP8 window rows [n, 584] u8."""
    rows = _c(rows_bf16, np.uint16)
    n = rows.shape[0]
    out = np.empty((n, swa_fp8_row_bytes()), np.uint8)
    lib().csa2o_swa_fp8_pack(_p(rows), n, _p(out))
    return out


def dequant_swa_fp8(rows8):
    rows8 = _c(rows8, np.uint8)
    out = np.empty((rows8.shape[0], D_LAT), np.float64)
    for r in range(rows8.shape[0]):
        lib().csa2o_dequant_swa_fp8(_p(rows8[r]), _p(out[r]))
    return out


def sparse_attn_swa_fp8(q_bf16, kv_cache, q_base, topk, swa8, swa_start, swa_len, swa_ring: int = 0,
                        scale: float = 1.0 / np.sqrt(512.0)):
    q = _c(q_bf16, np.uint16)
    n_q = q.shape[0]
    cache = _c(kv_cache, np.uint8)
    base = _c(q_base, np.int64)
    tk = _c(topk, np.int32)
    K = tk.shape[1]
    w8 = _c(swa8, np.uint8)
    ss = _c(swa_start, np.int64)
    sl = _c(swa_len, np.int32)
    out = np.empty((n_q, N_HEADS, D_LAT), np.float32)
    lse = np.empty((n_q, N_HEADS), np.float32)
    lib().csa2o_sparse_attn_swa_fp8(_p(q), _p(cache), _p(base), _p(tk), K, _p(w8), int(swa_ring), _p(ss), _p(sl),
                                    float(scale), _p(out), _p(lse), n_q)
    return out, lse
