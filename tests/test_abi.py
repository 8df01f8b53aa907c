"""CPU checks of the C-ABI library: it loads, exports every symbol the header declares,
and its host-side argument validation returns the documented status codes before any
launch.  No GPU compute is called."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fp4_kv_cache_csa2_amd", "libcsa2.so")
HEADER = os.path.join(ROOT, "include", "csa2.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libcsa2.so is not built")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(lib, s), f"missing export {s}"


def test_binding_names_match_header():
    from fp4_kv_cache_csa2_amd import csa2
    assert sorted(csa2.SYMBOLS) == declared_symbols()
    for name in ("rope_table", "compress_pack", "index_score", "block_topk", "sparse_attn"):
        assert callable(getattr(csa2, name))


def test_version_and_status_strings(lib):
    lib.csa2_status_string.restype = ctypes.c_char_p
    assert lib.csa2_abi_version() == 5
    for st in (0, -1, -2, -3, -4):
        assert lib.csa2_status_string(st)


def test_host_validation_rejects_before_launch(lib):
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.csa2_compress_pack.argtypes = [vp, i64, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.csa2_index_score.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.csa2_block_topk.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.csa2_sparse_attn.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, f32, vp, vp, i32, vp, sz, vp]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.csa2_compress_pack(fake, 4, 3, fake, 0, fake, fake, fake, fake, None) == -2
    assert lib.csa2_compress_pack(fake, -1, 2, fake, 0, fake, fake, fake, fake, None) == -1
    assert lib.csa2_compress_pack(None, 4, 2, fake, 0, fake, fake, fake, fake, None) == -1
    assert lib.csa2_compress_pack(fake, 4, 2, fake, 2, fake, fake, fake, fake, None) == -1  # per_token_w 0 or 1
    assert lib.csa2_compress_pack(fake, 0, 2, None, 0, None, None, None, None, None) == 0
    assert lib.csa2_index_score(fake, fake, fake, fake, fake, fake, 4096, 1, 8 * 4096, fake, None, None) == -2
    assert lib.csa2_index_score(fake, fake, fake, fake, fake, fake, 16, 1, 100, fake, None, None) == -1
    assert lib.csa2_index_score(None, fake, fake, fake, fake, None, 0, 1, 100, fake, None, None) == -1
    assert lib.csa2_block_topk(fake, None, 1, 100, fake, None, 4, 2048, 512, None, fake, None, 0, None) == -2
    assert lib.csa2_block_topk(fake, None, 1, 100, fake, None, 8, 2048, 513, None, fake, None, 0, None) == -2
    assert lib.csa2_block_topk(fake, None, 1, 200000, fake, None, 8, 2048, 512, None, fake, None, 0, None) == -3
    # a Full-mode Top-K needs M - 1 >= K (the global Top-K is the Top-K inside the pool only then)
    assert lib.csa2_block_topk(fake, None, 1, 200000, fake, None, 8, 64, 64, fake, fake, fake, 1 << 30, None) == -2
    assert lib.csa2_block_topk(fake, None, 1, 200000, fake, None, 8, 65, 64, fake, fake, None, 0, None) == -3
    assert lib.csa2_sparse_attn(fake, fake, fake, fake, 600, fake, fake, fake, 0.04, fake, None, 1,
                                None, 0, None) == -2
    assert lib.csa2_sparse_attn(fake, fake, fake, fake, 512, fake, fake, fake, 0.04, fake, None, 1,
                                None, 0, None) == -3
    assert lib.csa2_sparse_attn(ctypes.c_void_p((1 << 20) + 8), fake, fake, fake, 512, fake, fake, fake, 0.04, fake,
                                None, 1, fake, 1 << 30, None) == -1  # q not 16-B aligned
    assert lib.csa2_sparse_attn_workspace(4, 512) > 0  # small batches split a query's keys
    assert lib.csa2_sparse_attn_workspace(1 << 16, 512) == 0  # large ones do not
    assert lib.csa2_sparse_attn_workspace(128, 512) > 0 and lib.csa2_sparse_attn_workspace(129, 512) == 0


def test_fp8_window_entry_points_validate_before_launch(lib):
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.csa2_swa_pack_fp8.argtypes = [vp, i64, vp, vp, vp]
    lib.csa2_sparse_attn_swa_fp8.argtypes = [vp, vp, vp, vp, i32, vp, i64, vp, vp, f32, vp, vp, i32, vp, sz, vp]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.csa2_swa_pack_fp8(fake, -1, None, fake, None) == -1
    assert lib.csa2_swa_pack_fp8(fake, 0, None, None, None) == 0
    assert lib.csa2_swa_pack_fp8(ctypes.c_void_p((1 << 20) + 8), 4, None, fake, None) == -1  # rows not 16-B aligned
    assert lib.csa2_swa_pack_fp8(fake, 4, None, ctypes.c_void_p((1 << 20) + 4), None) == -1  # out not 8-B aligned
    attn = lib.csa2_sparse_attn_swa_fp8
    assert attn(fake, fake, fake, fake, 600, fake, 0, fake, fake, 0.04, fake, None, 1, None, 0, None) == -2
    assert attn(fake, fake, fake, fake, 512, fake, 64, fake, fake, 0.04, fake, None, 1, None, 0, None) == -1
    assert attn(fake, fake, fake, fake, 512, fake, -1, fake, fake, 0.04, fake, None, 1, None, 0, None) == -1
    assert attn(fake, fake, fake, fake, 512, ctypes.c_void_p((1 << 20) + 4), 0, fake, fake, 0.04, fake, None, 1,
                None, 0, None) == -1
    assert attn(fake, fake, fake, fake, 512, fake, 128, fake, fake, 0.04, fake, None, 1, None, 0, None) == -3


def test_rescore_selection_and_maxima_only_scan_validate_before_launch(lib):
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    f = lib.csa2_block_topk_rescore
    f.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.csa2_block_topk_rescore_workspace.argtypes = [i32, i32, i32, i32]
    lib.csa2_block_topk_rescore_workspace.restype = sz
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    odd = ctypes.c_void_p((1 << 20) + 4)
    need = lib.csa2_block_topk_rescore_workspace(4, 1 << 19, 2048, 512)
    # every list-B segment holds its whole slice: 64 workgroups x 8192 slots x 8 B per query
    assert need >= 4 * 64 * 8192 * 8
    assert need > lib.csa2_block_topk_rescore_workspace(1, 1 << 19, 2048, 512)
    args = [fake, 4, 1 << 19, fake, fake, fake, fake, fake, 2048, 512, fake, fake, fake, need, None]
    assert f(*args[:13], 16, None) == -3  # workspace too small
    assert f(*[None] + args[1:]) == -1  # block_max missing
    assert f(*args[:4], None, *args[5:]) == -1  # query missing
    assert f(*args[:11], None, *args[12:]) == -1  # topk_out required
    assert f(*args[:4], odd, *args[5:]) == -1  # q not 16-B aligned
    assert f(*args[:6], odd, *args[7:]) == -1  # idx_cache not 16-B aligned
    assert f(*args[:8], 4096, *args[9:]) == -2  # M > 2048
    assert f(*args[:9], 513, *args[10:]) == -2  # K > 512
    assert f(*args[:2], (1 << 23) + 8, *args[3:]) == -2  # rows longer than 2^23 entries
    assert f(None, 0, 0, None, None, None, None, None, 2048, 512, None, None, None, 0, None) == 0  # nothing to do
    # the fused scan: scores may be NULL only with the bf16 query and the block maxima
    for name in ("csa2_append_index_score", "csa2_append_index_score_fp4q", "csa2_append_index_score_packq"):
        g = getattr(lib, name)
        g.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp]
        a = [fake, 2, fake, 0, fake, fake, fake, fake, fake, fake, fake, fake, 4, 1 << 19]
        assert g(*a, None, None, None) == -1, name  # neither scores nor block maxima
        if name != "csa2_append_index_score":
            assert g(*a, None, fake, None) == -1, name  # the MXFP4-query scans write scores


def test_compress_append_validates_before_launch(lib):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.csa2_compress_append.argtypes = [vp, i64, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.csa2_compress_append(fake, 4, 1, None, 0, fake, fake, None, fake, fake, None) == -1  # no rows
    assert lib.csa2_compress_append(fake, 4, 3, fake, 0, fake, fake, fake, fake, fake, None) == -2
    assert lib.csa2_compress_append(fake, 4, 1, None, 0, fake, fake, ctypes.c_void_p((1 << 20) + 4), fake, fake,
                                    None) == -1  # rows not 8-B aligned
    assert lib.csa2_compress_append(fake, 4, 2, fake, -1, fake, fake, fake, fake, fake, None) == -1
    assert lib.csa2_compress_append(fake, 0, 1, None, 0, None, None, None, None, None, None) == 0


def test_fp4_query_entry_points_validate_before_launch(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.csa2_quantize_q_mxfp4.argtypes = [vp, i64, vp, vp]
    lib.csa2_index_score_fp4q.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.csa2_quantize_q_mxfp4(fake, -1, fake, None) == -1
    assert lib.csa2_quantize_q_mxfp4(fake, 0, None, None) == 0
    assert lib.csa2_quantize_q_mxfp4(None, 4, fake, None) == -1
    assert lib.csa2_quantize_q_mxfp4(ctypes.c_void_p((1 << 20) + 8), 4, fake, None) == -1  # q not 16-B aligned
    assert lib.csa2_quantize_q_mxfp4(fake, 4, ctypes.c_void_p((1 << 20) + 2), None) == -1  # out not 4-B aligned
    score = lib.csa2_index_score_fp4q
    assert score(fake, fake, fake, fake, fake, fake, 4096, 1, 8 * 4096, fake, None, None) == -2
    assert score(fake, fake, fake, fake, fake, fake, 16, 1, 100, fake, None, None) == -1
    assert score(None, fake, fake, fake, fake, None, 0, 1, 100, fake, None, None) == -1
    assert score(ctypes.c_void_p((1 << 20) + 2), fake, fake, fake, fake, None, 0, 1, 100, fake, None, None) == -1
    assert score(fake, fake, ctypes.c_void_p((1 << 20) + 4), fake, fake, None, 0, 1, 100, fake, None, None) == -1
    assert score(fake, fake, fake, fake, fake, None, 0, 0, 100, fake, None, None) == 0


def test_hisa_entry_points_validate_before_launch(lib):
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.csa2_block_mean_pack.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp]
    lib.csa2_block_topk.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    mean = lib.csa2_block_mean_pack
    assert mean(fake, fake, fake, None, -1, 4, fake, fake, None) == -1
    assert mean(fake, fake, fake, None, 2, -1, fake, fake, None) == -1
    assert mean(fake, fake, fake, None, 0, 4, fake, fake, None) == 0
    assert mean(None, fake, fake, None, 2, 4, fake, fake, None) == -1
    assert mean(fake, fake, fake, None, 2, 4, None, fake, None) == -1
    assert mean(ctypes.c_void_p((1 << 20) + 2), fake, fake, None, 2, 4, fake, fake, None) == -1
    assert mean(fake, fake, fake, None, 70000, 4, fake, fake, None) == -2
    topk = lib.csa2_block_topk
    # pool-only mode needs block scores and a pool output; scores may be NULL
    assert topk(None, None, 1, 800, fake, None, 8, 64, 16, fake, None, fake, 1 << 20, None) == -1
    assert topk(None, fake, 1, 800, fake, None, 8, 64, 16, None, None, fake, 1 << 20, None) == -1
    assert topk(None, fake, 1, 800, fake, fake, 8, 64, 16, None, None, fake, 1 << 20, None) == -1
    assert topk(None, fake, 1, 800, fake, None, 8, 64, 16, fake, fake, fake, 1 << 20, None) == -1  # Top-K needs scores
    assert topk(None, fake, 1, 800, fake, None, 8, 64, 16, fake, None, None, 0, None) == -3


def test_append_index_entry_points_validate_before_launch(lib):
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    f = 1 << 20  # never dereferenced: validation fails first
    for name, q_align in (("csa2_append_index_score", 16), ("csa2_append_index_score_fp4q", 4),
                          ("csa2_append_index_score_packq", 16)):
        fn = getattr(lib, name)
        fn.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp]

        def call(latent=f, m=2, pool_w=f, per_token=0, rope=f, w=f, kv=f, ix=f, q=f, hw=f, base=f, nvis=f, n_q=4,
                 width=1 << 19, scores=f, bmax=f):
            return fn(latent, m, pool_w, per_token, rope, w, kv, ix, q, hw, base, nvis, n_q, width, scores, bmax, None)

        assert call(n_q=0, latent=None, pool_w=None, q=None) == 0
        assert call(n_q=-1) == -1
        assert call(m=3) == -2
        assert call(width=0) == -1
        assert call(scores=None, bmax=None) == -1
        if name != "csa2_append_index_score":  # only the bf16-query scan may write block maxima alone
            assert call(scores=None) == -1
        assert call(pool_w=None) == -1
        assert call(n_q=70000) == -2
        assert call(width=(1 << 23) + 1) == -2
        assert call(latent=f + 2) == -1
        assert call(ix=f + 4) == -1
        assert call(q=f + q_align // 2) == -1
        assert call(bmax=f + 2) == -1
        assert call(per_token=3) == -1


def test_append_mean_index_entry_points_validate_before_launch(lib):
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    f = 1 << 20  # never dereferenced: validation fails first
    for name, q_align in (("csa2_append_mean_index_score", 16), ("csa2_append_mean_index_score_fp4q", 4)):
        fn = getattr(lib, name)
        fn.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp,
                       vp]

        def call(latent=f, m=2, pool_w=f, per_token=0, rope=f, w=f, kv=f, ix=f, mc=f, mbase=f, q=f, hw=f, base=f,
                 nvis=f, n_q=4, width=1 << 16, scores=f, bmax=f):
            return fn(latent, m, pool_w, per_token, rope, w, kv, ix, mc, mbase, q, hw, base, nvis, n_q, width, scores,
                      bmax, None)

        assert call(n_q=0, latent=None, mc=None, q=None) == 0
        assert call(n_q=-1) == -1
        assert call(m=0) == -2
        assert call(width=0) == -1
        assert call(mc=None) == -1
        assert call(mbase=None) == -1
        assert call(mc=f + 4) == -1
        assert call(pool_w=None) == -1
        assert call(n_q=70000) == -2
        assert call(width=(1 << 23) + 1) == -2
        assert call(ix=f + 4) == -1
        assert call(q=f + q_align // 2) == -1
        assert call(scores=f + 2) == -1
        assert call(per_token=2) == -1


def test_block_topk_noalloc_validates_before_launch(lib):
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    fn = lib.csa2_block_topk_noalloc
    fn.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, vp]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert fn(fake, None, -1, 100, fake, None, 8, 2048, 512, None, fake, None) == -1
    assert fn(fake, None, 1, 100, fake, None, 4, 2048, 512, None, fake, None) == -2
    assert fn(fake, None, 1, 100, fake, None, 8, 2048, 513, None, fake, None) == -2
    assert fn(None, None, 1, 100, fake, None, 8, 2048, 512, None, fake, None) == -1
    assert fn(fake, None, 0, 100, fake, None, 8, 2048, 512, None, fake, None) == 0
    # larger than the fixed array (4096 prefill rows): rejected on the host, nothing launched
    assert fn(fake, None, 4096, 34816, fake, None, 8, 2048, 512, None, fake, None) == -5
    lib.csa2_status_string.restype = ctypes.c_char_p
    assert b"scratch" in lib.csa2_status_string(-5)

