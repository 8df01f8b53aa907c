"""Thin Python binding over libcsa2.so (the C ABI declared in include/csa2.h).

Argument marshalling only: every step of the path runs in the HIP kernels.  Tensors are
torch tensors on the ROCm device; calls are enqueued on torch's current stream (or the
stream passed in).  Every wrapper checks the dtype, device, contiguity and shape of each
tensor it passes against the sizes of the call (n_q, width, M, K, ...) and raises
ValueError before anything is launched, so no kernel reads or writes past a tensor it was
given.  Index values held inside device tensors (cache rows, entry ids) are the caller's
to keep in range: checking them would need a device synchronisation per call.  Tensors the
binding allocates (outputs not given, workspaces) are allocated on the launch stream.
There is no CPU fallback: if libcsa2.so is missing or cannot be loaded, importing this
module raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libcsa2.so not built at {LIB_PATH}: run `python -m fp4_kv_cache_csa2_amd.build` "
                      "(or __graft_entry__.build()) first")

_L = ctypes.CDLL(LIB_PATH)
_vp, _i32, _i64, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                     ctypes.c_double, ctypes.c_size_t)
_L.csa2_abi_version.restype = ctypes.c_int
_L.csa2_status_string.argtypes = [ctypes.c_int]
_L.csa2_status_string.restype = ctypes.c_char_p
_L.csa2_rope_table.argtypes = [_vp, _i64, _f64, _vp]
_L.csa2_compress_pack.argtypes = [_vp, _i64, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp]
_L.csa2_compress_append.argtypes = [_vp, _i64, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp]
_L.csa2_index_score.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]
_L.csa2_quantize_q_mxfp4.argtypes = [_vp, _i64, _vp, _vp]
_L.csa2_index_score_fp4q.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]
_L.csa2_block_mean_pack.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp]
_L.csa2_append_index_score.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _i32, _i32, _vp, _vp, _vp]
_L.csa2_append_index_score_fp4q.argtypes = _L.csa2_append_index_score.argtypes
_L.csa2_append_index_score_sel.argtypes = _L.csa2_append_index_score.argtypes[:-1] + [_vp, _sz, _vp]
_L.csa2_append_index_score_packq.argtypes = _L.csa2_append_index_score.argtypes
_L.csa2_append_mean_index_score.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp]
_L.csa2_append_mean_index_score_fp4q.argtypes = _L.csa2_append_mean_index_score.argtypes
_L.csa2_block_topk_workspace.argtypes = [_i32, _i32, _i32, _i32]
_L.csa2_block_topk_workspace.restype = _sz
_L.csa2_block_topk.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
_L.csa2_block_topk_noalloc.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]
_L.csa2_block_topk_prebuilt.argtypes = [_vp, _vp, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
_L.csa2_block_topk_rescore_workspace.argtypes = [_i32, _i32, _i32, _i32]
_L.csa2_block_topk_rescore_workspace.restype = _sz
_L.csa2_block_topk_rescore.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz,
                                       _vp]
_L.csa2_sparse_attn_workspace.argtypes = [_i32, _i32]
_L.csa2_sparse_attn_workspace.restype = _sz
_L.csa2_sparse_attn.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _f32, _vp, _vp, _i32, _vp, _sz, _vp]
_L.csa2_swa_pack_fp8.argtypes = [_vp, _i64, _vp, _vp, _vp]
_L.csa2_sparse_attn_swa_fp8.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _i64, _vp, _vp, _f32, _vp, _vp, _i32, _vp,
                                        _sz, _vp]

SYMBOLS = ("csa2_abi_version", "csa2_status_string", "csa2_rope_table", "csa2_compress_pack", "csa2_compress_append",
           "csa2_index_score", "csa2_block_topk_workspace", "csa2_block_topk",
           "csa2_sparse_attn_workspace", "csa2_sparse_attn", "csa2_swa_pack_fp8", "csa2_sparse_attn_swa_fp8",
           "csa2_quantize_q_mxfp4", "csa2_index_score_fp4q", "csa2_block_mean_pack", "csa2_append_index_score",
           "csa2_append_index_score_fp4q", "csa2_append_index_score_packq", "csa2_append_mean_index_score",
           "csa2_append_mean_index_score_fp4q", "csa2_block_topk_noalloc", "csa2_block_topk_rescore_workspace",
           "csa2_block_topk_rescore", "csa2_append_index_score_sel", "csa2_block_topk_prebuilt")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 32 << 20
DEFAULT_SCALE = 512 ** -0.5
SWA_FP8_ROW_BYTES = 584
ROPE_THETA = 160000.0


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({_L.csa2_status_string(status).decode()})")
        self.status = status


def _check(fn: str, st: int) -> None:
    if st != OK:
        raise Csa2Error(fn, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context: tensors the binding makes are allocated on the launch stream."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _is_device(t) -> bool:
    return t.is_cuda


def _dev(t, dtype, name, shape=None):
    """Checks a device tensor: dtype, contiguity and, when given, its exact shape (a tuple
    whose None entries match any size)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
            want = tuple("*" if w is None else w for w in shape)
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")


def _need(t, name):
    if t is None:
        raise ValueError(f"{name} is required")


def _bytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def abi_version() -> int:
    return _L.csa2_abi_version()


def rope_table(pos, theta: float = ROPE_THETA) -> torch.Tensor:
    """Host cos/sin table [n, 64] (fp32, CPU tensor) for entry positions `pos` (CPU int64)."""
    pos = torch.as_tensor(pos, dtype=torch.int64).contiguous()
    out = torch.empty((pos.numel(), 64), dtype=torch.float32)
    _check("csa2_rope_table", _L.csa2_rope_table(_ptr(pos), pos.numel(), float(theta), _ptr(out)))
    return out


def _pool_weights(pool_w, m: int, n_rows: int) -> int:
    """Checks the pooling weights of n_rows latent rows: [m, 512] static (returns 0) or
    [n_rows, 512] per token (returns 1); m = 1 reads none and may pass None."""
    if pool_w is None:
        if m != 1:
            raise ValueError("pool_w is required when m > 1")
        return 0
    _dev(pool_w, torch.float32, "pool_w", (None, 512))
    if pool_w.shape[0] == m:
        return 0
    if pool_w.shape[0] == n_rows:
        return 1
    raise ValueError(f"pool_w must be [m, 512] (static) or [{n_rows}, 512] (one row per latent token), "
                     f"got {tuple(pool_w.shape)}")


def _latent_rows(latent, m: int) -> int:
    _dev(latent, torch.bfloat16, "latent", (None, 512))
    if m not in (1, 2):
        raise ValueError("m must be 1 or 2")
    if latent.shape[0] % m:
        raise ValueError("latent must hold complete groups of m rows")
    return latent.shape[0] // m


def _cache(t, name, row_bytes):
    _need(t, name)
    _dev(t, torch.uint8, name, (None, row_bytes))


# The indexer-K cache (and HISA's block-mean cache) is a tensor of tiles: uint8 [n_tiles, 2176],
# 32 entries per tile (include/csa2.h gives the byte layout); entry j lives in tile j // 32.
IDX_TILE_ENTRIES = 32
IDX_TILE_BYTES = 2176


def idx_tiles_for(n_entries: int) -> int:
    """Tiles an indexer-K cache needs to hold entries 0 .. n_entries - 1."""
    return (n_entries + IDX_TILE_ENTRIES - 1) // IDX_TILE_ENTRIES


def _idx_cache(t, name):
    _cache(t, name, IDX_TILE_BYTES)


def compress_pack(latent, m: int, pool_w, rope_cs, w_idx, kv_out=None, idx_out=None, stream=None):
    """latent bf16 [n*m, 512] -> (kv uint8 [n, 288], idx uint8 [idx_tiles_for(n), 2176]); outputs
    may be given (room for at least n entries).  pool_w: fp32 [m, 512], or [n*m, 512] for one
    weight row per token."""
    n = _latent_rows(latent, m)
    per_token = _pool_weights(pool_w, m, n * m)
    _dev(rope_cs, torch.float32, "rope_cs", (None, 64))
    _dev(w_idx, torch.bfloat16, "w_idx", (128, 512))
    with _on(stream):
        if kv_out is None:
            kv_out = torch.empty((n, 288), dtype=torch.uint8, device=latent.device)
        if idx_out is None:
            idx_out = torch.empty((idx_tiles_for(n), IDX_TILE_BYTES), dtype=torch.uint8, device=latent.device)
    _cache(kv_out, "kv_out", 288)
    _idx_cache(idx_out, "idx_out")
    if rope_cs.shape[0] < n or kv_out.shape[0] < n or idx_out.shape[0] * IDX_TILE_ENTRIES < n:
        raise ValueError("rope_cs, kv_out and idx_out need room for every entry")
    _check("csa2_compress_pack", _L.csa2_compress_pack(
        _ptr(latent), n, m, _ptr(pool_w), per_token, _ptr(rope_cs), _ptr(w_idx), _ptr(kv_out), _ptr(idx_out),
        _stream(stream)))
    return kv_out, idx_out


def compress_append(latent, m: int, pool_w, rope_cs, w_idx, dst_rows, kv_cache, idx_cache, stream=None):
    """Pack entries from latent bf16 [n*m, 512] into cache rows dst_rows (int64 [n], -1 drops;
    every row must lie inside both caches)."""
    n = _latent_rows(latent, m)
    per_token = _pool_weights(pool_w, m, n * m)
    _dev(rope_cs, torch.float32, "rope_cs", (None, 64))
    _dev(w_idx, torch.bfloat16, "w_idx", (128, 512))
    _need(dst_rows, "dst_rows")
    _dev(dst_rows, torch.int64, "dst_rows", (n,))
    _cache(kv_cache, "kv_cache", 288)
    _idx_cache(idx_cache, "idx_cache")
    if rope_cs.shape[0] < n:
        raise ValueError("rope_cs must cover every new entry")
    _check("csa2_compress_append", _L.csa2_compress_append(
        _ptr(latent), n, m, _ptr(pool_w), per_token, _ptr(rope_cs), _ptr(w_idx), _ptr(dst_rows), _ptr(kv_cache),
        _ptr(idx_cache), _stream(stream)))


def _query_rows(q_base, q_nvis, n_q):
    _need(q_base, "q_base")
    _need(q_nvis, "q_nvis")
    _dev(q_base, torch.int64, "q_base", (n_q,))
    _dev(q_nvis, torch.int32, "q_nvis", (n_q,))


def _score_outputs(scores, block_max, want_block_max, n_q, width, dev, stream, full_mode=True, want_scores=True):
    with _on(stream):
        if scores is None and want_scores:
            scores = torch.empty((n_q, width), dtype=torch.float32, device=dev)
        if block_max is None and want_block_max and full_mode:
            block_max = torch.empty((n_q, (width + 7) // 8), dtype=torch.float32, device=dev)
    _dev(scores, torch.float32, "scores", (n_q, width))
    if block_max is not None and not full_mode:
        raise ValueError("block_max is written in Full mode only")
    _dev(block_max, torch.float32, "block_max", (n_q, (width + 7) // 8))
    return scores, block_max


def _index_args(q, q_kind, head_w, idx_cache, q_base, q_nvis, width, pool_blocks):
    if q_kind == "fp4":
        _dev(q, torch.uint8, "q_fp4", (None, 32, 68))
    else:
        _dev(q, torch.bfloat16, "q_idx", (None, 32, 128))
    n_q = q.shape[0]
    _dev(head_w, torch.float32, "head_w", (n_q, 32))
    _idx_cache(idx_cache, "idx_cache")
    _query_rows(q_base, q_nvis, n_q)
    M = 0
    if pool_blocks is not None:
        _dev(pool_blocks, torch.int32, "pool_blocks", (n_q, None))
        M = pool_blocks.shape[1]
        if width != 8 * M:
            raise ValueError(f"candidate mode scores 8 slots per pool block: width must be {8 * M}")
    if width < 0:
        raise ValueError("width must be >= 0")
    return n_q, M


def index_score(q_idx, head_w, idx_cache, q_base, q_nvis, width: int, pool_blocks=None,
                scores=None, block_max=None, want_block_max: bool = True, stream=None):
    """Indexer scores [n_q, width] (+ block maxima [n_q, ceil(width/8)] in Full mode)."""
    n_q, M = _index_args(q_idx, "bf16", head_w, idx_cache, q_base, q_nvis, width, pool_blocks)
    scores, block_max = _score_outputs(scores, block_max, want_block_max, n_q, width, q_idx.device, stream,
                                       full_mode=pool_blocks is None)
    _check("csa2_index_score", _L.csa2_index_score(
        _ptr(q_idx), _ptr(head_w), _ptr(idx_cache), _ptr(q_base), _ptr(q_nvis), _ptr(pool_blocks),
        M, n_q, width, _ptr(scores), _ptr(block_max), _stream(stream)))
    return scores, block_max


def _append_args(latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, n_q):
    n = _latent_rows(latent, m)
    if n != n_q:
        raise ValueError("latent must hold m rows per query")
    per_token = _pool_weights(pool_w, m, n_q * m)
    _dev(rope_cs, torch.float32, "rope_cs", (None, 64))
    if rope_cs.shape[0] < n_q:
        raise ValueError("rope_cs must cover every new entry")
    _dev(w_idx, torch.bfloat16, "w_idx", (128, 512))
    _cache(kv_cache, "kv_cache", 288)
    _idx_cache(idx_cache, "idx_cache")
    return per_token


def append_index_score(latent, m: int, pool_w, rope_cs, w_idx, kv_cache, idx_cache, q_idx, head_w, q_base, q_nvis,
                       width: int, scores=None, block_max=None, want_block_max: bool = True, stream=None,
                       pack_q: bool = False, want_scores: bool = True, sel_workspace=None):
    """Appends query t's newest entry (latent bf16 [n_q*m, 512]) at cache row
    q_base[t] + q_nvis[t] - 1, then scores every visible entry: compress_append followed by
    Full-mode index_score, in one launch.  q_idx is bf16 [n_q, 32, 128] or MXFP4 uint8
    [n_q, 32, 68] (from quantize_q_mxfp4); pack_q=True with a bf16 q_idx packs it to MXFP4
    inside the launch (quantize_q_mxfp4 followed by the MXFP4-query call).  pool_w: fp32
    [m, 512], or [n_q*m, 512] for one weight row per latent token.  want_scores=False (bf16
    query): the block maxima alone are written and scores comes back None (the selection then
    uses block_topk_rescore).  sel_workspace (bf16 query): the workspace of the block_topk
    call that follows (histogram region zeroed, as every block_topk call leaves it), into
    which the launch also counts the older blocks' maxima; that call then passes
    hist_ready=True and skips its first pass."""
    fp4 = isinstance(q_idx, torch.Tensor) and q_idx.dtype == torch.uint8
    if sel_workspace is not None and (fp4 or pack_q or not want_block_max):
        raise ValueError("sel_workspace takes a bf16 q_idx and the block maxima")
    if pack_q and fp4:
        raise ValueError("pack_q takes a bf16 q_idx")
    if not want_scores and (fp4 or pack_q or scores is not None or not want_block_max):
        raise ValueError("want_scores=False takes a bf16 q_idx, no scores buffer and the block maxima")
    n_q, _ = _index_args(q_idx, "fp4" if fp4 else "bf16", head_w, idx_cache, q_base, q_nvis, width, None)
    per_token = _append_args(latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, n_q)
    scores, block_max = _score_outputs(scores, block_max, want_block_max, n_q, width, q_idx.device, stream,
                                       want_scores=want_scores)
    if sel_workspace is not None:
        _dev(sel_workspace, sel_workspace.dtype, "sel_workspace")
        if _bytes(sel_workspace) < n_q * 4096 * 4:
            raise ValueError(f"sel_workspace: at least {n_q * 4096 * 4} bytes (the histogram rows), "
                             f"got {_bytes(sel_workspace)}")
        _check("csa2_append_index_score_sel", _L.csa2_append_index_score_sel(
            _ptr(latent), m, _ptr(pool_w), per_token, _ptr(rope_cs), _ptr(w_idx), _ptr(kv_cache), _ptr(idx_cache),
            _ptr(q_idx), _ptr(head_w), _ptr(q_base), _ptr(q_nvis), n_q, width, _ptr(scores), _ptr(block_max),
            _ptr(sel_workspace), _bytes(sel_workspace), _stream(stream)))
        return scores, block_max
    name = "csa2_append_index_score" + ("_fp4q" if fp4 else "_packq" if pack_q else "")
    fn = getattr(_L, name)
    _check(name, fn(
        _ptr(latent), m, _ptr(pool_w), per_token, _ptr(rope_cs), _ptr(w_idx), _ptr(kv_cache), _ptr(idx_cache),
        _ptr(q_idx), _ptr(head_w), _ptr(q_base), _ptr(q_nvis), n_q, width, _ptr(scores), _ptr(block_max),
        _stream(stream)))
    return scores, block_max


def append_mean_index_score(latent, m: int, pool_w, rope_cs, w_idx, kv_cache, idx_cache, mean_cache, mean_base,
                            q_idx, head_w, q_base, q_nvis, width: int, scores=None, block_max=None,
                            want_block_max: bool = False, stream=None):
    """HISA's decode step in one launch: appends query t's newest entry as append_index_score
    does, re-packs the mean record of the block holding it (mean_cache row
    mean_base[t] + (q_nvis[t] - 1) // 8), then scores the ceil(q_nvis[t] / 8) visible block
    means: compress_append, block_mean_pack and index_score over mean_cache."""
    fp4 = isinstance(q_idx, torch.Tensor) and q_idx.dtype == torch.uint8
    n_q, _ = _index_args(q_idx, "fp4" if fp4 else "bf16", head_w, idx_cache, q_base, q_nvis, width, None)
    per_token = _append_args(latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, n_q)
    _idx_cache(mean_cache, "mean_cache")
    _need(mean_base, "mean_base")
    _dev(mean_base, torch.int64, "mean_base", (n_q,))
    scores, block_max = _score_outputs(scores, block_max, want_block_max, n_q, width, q_idx.device, stream)
    fn = _L.csa2_append_mean_index_score_fp4q if fp4 else _L.csa2_append_mean_index_score
    _check("csa2_append_mean_index_score" + ("_fp4q" if fp4 else ""), fn(
        _ptr(latent), m, _ptr(pool_w), per_token, _ptr(rope_cs), _ptr(w_idx), _ptr(kv_cache), _ptr(idx_cache),
        _ptr(mean_cache), _ptr(mean_base), _ptr(q_idx), _ptr(head_w), _ptr(q_base), _ptr(q_nvis), n_q, width,
        _ptr(scores), _ptr(block_max), _stream(stream)))
    return scores, block_max


def quantize_q_mxfp4(q_idx, out=None, stream=None):
    """bf16 head vectors [..., 128] -> MXFP4 records uint8 [..., 68] (the indexer-K format)."""
    _dev(q_idx, torch.bfloat16, "q_idx")
    if q_idx.dim() < 1 or q_idx.shape[-1] != 128:
        raise ValueError("q_idx must end in 128 channels")
    n_vec = q_idx.numel() // 128
    with _on(stream):
        if out is None:
            out = torch.empty((*q_idx.shape[:-1], 68), dtype=torch.uint8, device=q_idx.device)
    _dev(out, torch.uint8, "out", (*q_idx.shape[:-1], 68))
    _check("csa2_quantize_q_mxfp4", _L.csa2_quantize_q_mxfp4(_ptr(q_idx), n_vec, _ptr(out), _stream(stream)))
    return out


def index_score_fp4q(q_fp4, head_w, idx_cache, q_base, q_nvis, width: int, pool_blocks=None,
                     scores=None, block_max=None, want_block_max: bool = True, stream=None):
    """index_score with MXFP4 queries q_fp4 uint8 [n_q, 32, 68] (from quantize_q_mxfp4)."""
    n_q, M = _index_args(q_fp4, "fp4", head_w, idx_cache, q_base, q_nvis, width, pool_blocks)
    scores, block_max = _score_outputs(scores, block_max, want_block_max, n_q, width, q_fp4.device, stream,
                                       full_mode=pool_blocks is None)
    _check("csa2_index_score_fp4q", _L.csa2_index_score_fp4q(
        _ptr(q_fp4), _ptr(head_w), _ptr(idx_cache), _ptr(q_base), _ptr(q_nvis), _ptr(pool_blocks),
        M, n_q, width, _ptr(scores), _ptr(block_max), _stream(stream)))
    return scores, block_max


def block_topk_workspace(n_q: int, width: int, M: int, K: int) -> int:
    return int(_L.csa2_block_topk_workspace(n_q, width, M, K))


def block_topk(scores, q_nvis, K: int = 512, M: int = 2048, block_max=None, pool_blocks=None,
               want_pool: bool = True, pool_out=None, topk_out=None, workspace=None, stream=None,
               want_topk: bool = True, hist_ready: bool = False):
    """(pool [n_q, M] or None, topk [n_q, K] or None): Full mode when pool_blocks is None.
    want_topk=False is the pool-only mode: the pool from block_max [n_q, nbw] (the caller's
    block scores); scores may then be None (the row width is 8 * nbw).  A given workspace
    must hold block_topk_workspace(...) bytes and start zeroed (every call leaves it so).
    hist_ready=True (Full mode, block_max and workspace given): append_index_score with
    sel_workspace=workspace already counted the first pass (csa2_block_topk_prebuilt)."""
    if hist_ready and (pool_blocks is not None or block_max is None or workspace is None):
        raise ValueError("hist_ready takes Full mode, block_max and the workspace the counts went into")
    _dev(scores, torch.float32, "scores", (None, None))
    if scores is not None:
        n_q, width = scores.shape
        dev = scores.device
    else:
        if want_topk or block_max is None:
            raise ValueError("scores may be None only in pool-only mode (want_topk=False, block_max given)")
        _dev(block_max, torch.float32, "block_max", (None, None))
        n_q, width = block_max.shape[0], 8 * block_max.shape[1]
        dev = block_max.device
    _need(q_nvis, "q_nvis")
    _dev(q_nvis, torch.int32, "q_nvis", (n_q,))
    _dev(block_max, torch.float32, "block_max", (n_q, (width + 7) // 8))
    if pool_blocks is not None:
        _dev(pool_blocks, torch.int32, "pool_blocks", (n_q, None))
        M = pool_blocks.shape[1]
        want_pool = False
        if width != 8 * M or block_max is not None or pool_out is not None:
            raise ValueError("candidate mode: scores [n_q, 8 * M], no block_max and no pool output")
    with _on(stream):
        if pool_out is None and want_pool:
            pool_out = torch.empty((n_q, M), dtype=torch.int32, device=dev)
        if topk_out is None and want_topk:
            topk_out = torch.empty((n_q, K), dtype=torch.int32, device=dev)
        need = block_topk_workspace(n_q, width, M, K)
        if workspace is None:
            # the histogram region must start zeroed; every call leaves it zeroed
            workspace = torch.zeros(max(need, 4), dtype=torch.uint8, device=dev)
    _dev(pool_out, torch.int32, "pool_out", (n_q, M))
    _dev(topk_out, torch.int32, "topk_out", (n_q, K))
    _dev(workspace, workspace.dtype, "workspace")
    if hist_ready:
        if _bytes(workspace) < need:
            raise ValueError(f"workspace: block_topk_workspace gives {need} bytes, got {_bytes(workspace)}")
        _check("csa2_block_topk_prebuilt", _L.csa2_block_topk_prebuilt(
            _ptr(scores), _ptr(block_max), n_q, width, _ptr(q_nvis), 8, M, K, _ptr(pool_out), _ptr(topk_out),
            _ptr(workspace), _bytes(workspace), _stream(stream)))
        return pool_out, topk_out
    _check("csa2_block_topk", _L.csa2_block_topk(
        _ptr(scores), _ptr(block_max), n_q, width, _ptr(q_nvis), _ptr(pool_blocks), 8, M, K,
        _ptr(pool_out), _ptr(topk_out), _ptr(workspace), _bytes(workspace), _stream(stream)))
    return pool_out, topk_out


def block_topk_noalloc(scores, q_nvis, K: int = 512, M: int = 2048, block_max=None, pool_blocks=None,
                       pool_out=None, topk_out=None, stream=None):
    """block_topk through the allocation-free entry point (the library's fixed scratch array,
    NOALLOC_SCRATCH_BYTES per GPU): the outputs must be given, so the call allocates nothing;
    pool_out None with topk_out given skips the pool, topk_out None is the pool-only mode.
    Calls that overlap in time on one GPU must not be issued."""
    if scores is not None:
        _dev(scores, torch.float32, "scores", (None, None))
        n_q, width = scores.shape
    else:
        _need(block_max, "block_max")
        _dev(block_max, torch.float32, "block_max", (None, None))
        n_q, width = block_max.shape[0], 8 * block_max.shape[1]
    _need(q_nvis, "q_nvis")
    _dev(q_nvis, torch.int32, "q_nvis", (n_q,))
    _dev(block_max, torch.float32, "block_max", (n_q, (width + 7) // 8))
    if pool_blocks is not None:
        _dev(pool_blocks, torch.int32, "pool_blocks", (n_q, None))
        M = pool_blocks.shape[1]
        if width != 8 * M or block_max is not None or pool_out is not None:
            raise ValueError("candidate mode: scores [n_q, 8 * M], no block_max and no pool output")
    if pool_out is None and topk_out is None:
        raise ValueError("give pool_out, topk_out or both")
    _dev(pool_out, torch.int32, "pool_out", (n_q, M))
    _dev(topk_out, torch.int32, "topk_out", (n_q, K))
    _check("csa2_block_topk_noalloc", _L.csa2_block_topk_noalloc(
        _ptr(scores), _ptr(block_max), n_q, width, _ptr(q_nvis), _ptr(pool_blocks), 8, M, K, _ptr(pool_out),
        _ptr(topk_out), _stream(stream)))
    return pool_out, topk_out


def block_mean_pack(idx_cache, seq_base, seq_n, n_blocks: int, mean_cache, mean_base, first_block=None,
                    stream=None):
    """HISA block-mean records of blocks first_block[s] .. + n_blocks - 1 into mean_cache."""
    _idx_cache(idx_cache, "idx_cache")
    _idx_cache(mean_cache, "mean_cache")
    _need(seq_base, "seq_base")
    n_seq = seq_base.numel()
    for t, name, dt in ((seq_base, "seq_base", torch.int64), (seq_n, "seq_n", torch.int32),
                        (mean_base, "mean_base", torch.int64), (first_block, "first_block", torch.int32)):
        if t is None and name != "first_block":
            raise ValueError(f"{name} is required")
        _dev(t, dt, name, (n_seq,))
    _check("csa2_block_mean_pack", _L.csa2_block_mean_pack(
        _ptr(idx_cache), _ptr(seq_base), _ptr(seq_n), _ptr(first_block), n_seq, n_blocks, _ptr(mean_cache),
        _ptr(mean_base), _stream(stream)))
    return mean_cache


def block_topk_rescore_workspace(n_q: int, width: int, M: int, K: int) -> int:
    return int(_L.csa2_block_topk_rescore_workspace(n_q, width, M, K))


def block_topk_rescore(block_max, q_nvis, q_idx, head_w, idx_cache, q_base, width: int, K: int = 512,
                       M: int = 2048, want_pool: bool = True, pool_out=None, topk_out=None, workspace=None,
                       stream=None):
    """(pool [n_q, M] or None, topk [n_q, K]): Full-mode selection from the block maxima
    [n_q, ceil(width/8)], re-scoring the candidate entries from the indexer cache (bf16
    q_idx [n_q, 32, 128], head_w [n_q, 32], idx_cache [n_tiles, 2176], q_base [n_q]); the result
    of block_topk on the score row the scan would have written.  A given workspace must hold
    block_topk_rescore_workspace(...) bytes and start zeroed (every call leaves it so)."""
    _need(block_max, "block_max")
    _dev(block_max, torch.float32, "block_max", (None, (width + 7) // 8))
    n_q = block_max.shape[0]
    dev = block_max.device
    _need(q_nvis, "q_nvis")
    _dev(q_nvis, torch.int32, "q_nvis", (n_q,))
    _index_args(q_idx, "bf16", head_w, idx_cache, q_base, q_nvis, width, None)
    if q_idx.shape[0] != n_q:
        raise ValueError("q_idx needs one query per block_max row")
    with _on(stream):
        if pool_out is None and want_pool:
            pool_out = torch.empty((n_q, M), dtype=torch.int32, device=dev)
        if topk_out is None:
            topk_out = torch.empty((n_q, K), dtype=torch.int32, device=dev)
        if workspace is None:  # the histogram region must start zeroed; every call leaves it zeroed
            workspace = torch.zeros(max(block_topk_rescore_workspace(n_q, width, M, K), 4), dtype=torch.uint8,
                                    device=dev)
    _dev(pool_out, torch.int32, "pool_out", (n_q, M))
    _dev(topk_out, torch.int32, "topk_out", (n_q, K))
    _dev(workspace, workspace.dtype, "workspace")
    _check("csa2_block_topk_rescore", _L.csa2_block_topk_rescore(
        _ptr(block_max), n_q, width, _ptr(q_nvis), _ptr(q_idx), _ptr(head_w), _ptr(idx_cache), _ptr(q_base), M, K,
        _ptr(pool_out), _ptr(topk_out), _ptr(workspace), _bytes(workspace), _stream(stream)))
    return pool_out, topk_out


def sparse_attn_workspace(n_q: int, K: int) -> int:
    return int(_L.csa2_sparse_attn_workspace(n_q, K))


def _attn_args(q, kv_cache, q_base, topk, swa_start, swa_len):
    _dev(q, torch.bfloat16, "q", (None, 64, 512))
    n_q = q.shape[0]
    _cache(kv_cache, "kv_cache", 288)
    _need(q_base, "q_base")
    _dev(q_base, torch.int64, "q_base", (n_q,))
    _need(topk, "topk")
    _dev(topk, torch.int32, "topk", (n_q, None))
    for t, name, dt in ((swa_start, "swa_start", torch.int64), (swa_len, "swa_len", torch.int32)):
        _need(t, name)
        _dev(t, dt, name, (n_q,))
    return n_q, topk.shape[1]


def _attn_outputs(out, lse, want_lse, workspace, n_q, K, dev, stream):
    with _on(stream):
        if out is None:
            out = torch.empty((n_q, 64, 512), dtype=torch.float32, device=dev)
        if lse is None and want_lse:
            lse = torch.empty((n_q, 64), dtype=torch.float32, device=dev)
        need = sparse_attn_workspace(n_q, K)
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(out, torch.float32, "out", (n_q, 64, 512))
    _dev(lse, torch.float32, "lse", (n_q, 64))
    if workspace is not None:
        _dev(workspace, workspace.dtype, "workspace")
    return out, lse, workspace


def sparse_attn(q, kv_cache, q_base, topk, swa, swa_start, swa_len, scale: float = DEFAULT_SCALE,
                out=None, lse=None, want_lse: bool = True, workspace=None, stream=None):
    """Attention output fp32 [n_q, 64, 512] (+ lse [n_q, 64])."""
    n_q, K = _attn_args(q, kv_cache, q_base, topk, swa_start, swa_len)
    _need(swa, "swa")
    _dev(swa, torch.bfloat16, "swa", (None, 512))
    out, lse, workspace = _attn_outputs(out, lse, want_lse, workspace, n_q, K, q.device, stream)
    _check("csa2_sparse_attn", _L.csa2_sparse_attn(
        _ptr(q), _ptr(kv_cache), _ptr(q_base), _ptr(topk), K, _ptr(swa), _ptr(swa_start), _ptr(swa_len),
        float(scale), _ptr(out), _ptr(lse), n_q, _ptr(workspace), _bytes(workspace), _stream(stream)))
    return out, lse


def swa_pack_fp8(rows, out=None, dst_rows=None, stream=None):
    """bf16 window rows [n, 512] -> FP8 window rows uint8 [n, 584] (or into `out` at dst_rows)."""
    _dev(rows, torch.bfloat16, "rows", (None, 512))
    n = rows.shape[0]
    _dev(dst_rows, torch.int64, "dst_rows", (n,))
    with _on(stream):
        if out is None:
            out = torch.empty((n, SWA_FP8_ROW_BYTES), dtype=torch.uint8, device=rows.device)
    _cache(out, "out", SWA_FP8_ROW_BYTES)
    if dst_rows is None and out.shape[0] < n:
        raise ValueError("out needs a row per input row")
    _check("csa2_swa_pack_fp8", _L.csa2_swa_pack_fp8(_ptr(rows), n, _ptr(dst_rows), _ptr(out), _stream(stream)))
    return out


def sparse_attn_swa_fp8(q, kv_cache, q_base, topk, swa8, swa_start, swa_len, swa_ring: int = 0,
                        scale: float = DEFAULT_SCALE, out=None, lse=None, want_lse: bool = True,
                        workspace=None, stream=None):
    """sparse_attn with the window read from FP8 window rows (optionally per-sequence rings)."""
    n_q, K = _attn_args(q, kv_cache, q_base, topk, swa_start, swa_len)
    _cache(swa8, "swa8", SWA_FP8_ROW_BYTES)
    out, lse, workspace = _attn_outputs(out, lse, want_lse, workspace, n_q, K, q.device, stream)
    _check("csa2_sparse_attn_swa_fp8", _L.csa2_sparse_attn_swa_fp8(
        _ptr(q), _ptr(kv_cache), _ptr(q_base), _ptr(topk), K, _ptr(swa8), int(swa_ring), _ptr(swa_start),
        _ptr(swa_len), float(scale), _ptr(out), _ptr(lse), n_q, _ptr(workspace), _bytes(workspace),
        _stream(stream)))
    return out, lse
