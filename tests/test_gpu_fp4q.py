"""GPU parity of the MXFP4 indexer query (the FP4 indexer Q of DeepSeek-V4's QAT): the query
packer bit-exact against the oracle, and the FP4-query scores (one-query decode kernel,
many-query prefill kernel, candidate mode) within the score tolerance of the oracle's
FP4-query scores, with block maxima equal to the maxima of the GPU's own scores.  The full
prefill chunk (4096 queries x <= 34816 entries) and one 1M-context decode query are
checked on sampled queries, including their Top-512."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth
from tests.gpu_util import bf16, check_scores, check_selection, dev, dev_ix, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_csa2_amd import csa2
    return csa2


def log(msg):
    print(msg, flush=True)


def _spread_q(seed, n_q):
    """q_idx ~ N(0,1)/sqrt(128) with every 32-channel group scaled by 2^[-20, 8): exercises
    every E8M0 code range the workloads can reach, plus zero groups and lone zeros."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_q, 32, 128)).astype(np.float32) / np.float32(np.sqrt(128.0))
    x *= (2.0 ** rng.integers(-20, 8, size=(n_q, 32, 4))).repeat(32, axis=2).astype(np.float32)
    x[0, 0, :32] = 0.0
    x[0, 1, 40] = 0.0
    return synth.f32_to_bf16_bits(x)


def _check_bmax(s, bm, width):
    n_q = s.shape[0]
    nbw = (width + 7) // 8
    pad = np.full((n_q, nbw * 8), -np.inf, np.float32)
    pad[:, :width] = s
    assert np.array_equal(bm, pad.reshape(n_q, nbw, 8).max(axis=2))


# ------------------------------------------------------------------ query packer
@pytest.mark.parametrize("n_q,seed", [(1, 1), (3, 2), (37, 3)])
def test_quantize_q_bit_exact(c, n_q, seed):
    log(f"quantize_q n_q={n_q} seed={seed}")
    qb = _spread_q(seed, n_q)
    ref = oracle.quantize_q_mxfp4(qb)
    got = host(c.quantize_q_mxfp4(bf16(qb)))
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), f"{np.sum(np.any(got != ref, axis=-1))} head records differ"


def test_quantize_q_edge_values(c):
    """Zero and negative-zero groups, bf16 subnormals, the largest bf16, infinities, NaN,
    exact E2M1 midpoints (ties to the even code) and values on the saturation band."""
    log("quantize_q edge values")
    x = np.zeros((2, 32, 128), np.float32)
    x[0, 1, :] = -0.0
    x[0, 2, :] = np.float32(2.0 ** -130) * np.arange(1, 129)     # subnormal bf16 group
    x[0, 3, :] = np.float32(3.3895314e38)                         # largest bf16
    x[0, 4, :] = 1.0
    x[0, 4, 7] = np.inf                                           # group holding +inf
    x[0, 5, 33] = -np.inf
    x[0, 6, :] = np.nan
    x[0, 6, 64:] = 1.0
    grid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    x[0, 7, :] = np.tile(np.concatenate([grid, -grid, [4.0, 7.0]]), 8)[:128]  # midpoints at X = 1 (amax 7 -> X = 1)
    x[0, 8, :] = np.tile(np.array([7.9, 6.0, -7.5, 3.0], np.float32), 32)   # (6X, 8X) clamps to 6X
    rng = np.random.default_rng(5)
    x[1] = rng.standard_normal((32, 128)).astype(np.float32) * 1e-3
    qb = synth.f32_to_bf16_bits(x)
    ref = oracle.quantize_q_mxfp4(qb)
    got = host(c.quantize_q_mxfp4(bf16(qb)))
    bad = np.argwhere(np.any(got != ref, axis=-1))
    assert bad.size == 0, f"records differ at {bad[:8].tolist()}"


# ------------------------------------------------------------------ scores
@pytest.mark.parametrize("n_q,n,width_pad,seed", [(1, 2048, 0, 5), (3, 1000, 77, 6), (4, 4096, 8, 7), (2, 33, 0, 8)])
def test_index_score_fp4q_full_mode(c, n_q, n, width_pad, seed):
    log(f"index_score_fp4q full n_q={n_q} n={n} seed={seed}")
    kv, ix = synth.random_caches(seed, n * n_q)
    d = synth.query_inputs(seed + 100, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.array([n - (7 * t) % max(n // 3, 1) for t in range(n_q)], np.int32)
    width = n + width_pad
    qf_ref = oracle.quantize_q_mxfp4(d.q_idx)
    ref = oracle.index_score_fp4q(qf_ref, d.head_w, ix, base, nvis, width)
    qf = c.quantize_q_mxfp4(bf16(d.q_idx))
    s, bm = c.index_score_fp4q(qf, dev(d.head_w), dev_ix(ix), dev(base), dev(nvis), width)
    torch.cuda.synchronize()
    assert np.array_equal(host(qf), qf_ref)
    s, bm = host(s), host(bm)
    check_scores(s, ref)
    _check_bmax(s, bm, width)


@pytest.mark.parametrize("shared", [True, False])
def test_index_score_fp4q_many_queries(c, shared):
    """Batches of >= 64 queries take the many-query FP4 kernel: one shared sequence with
    causal visibility (queries not a multiple of the 16 per workgroup, ragged last tile,
    queries that see nothing or one entry), or one sequence per query."""
    n_q = 72 if shared else 66
    n = 3001 if shared else 611
    log(f"index_score_fp4q many queries shared={shared} n_q={n_q} n={n}")
    kv, ix = synth.random_caches(51 if shared else 52, n if shared else n * n_q)
    d = synth.query_inputs(53, n_q)
    if shared:
        base = np.zeros(n_q, np.int64)
        nvis = np.array([n - 37 * t for t in range(n_q)], np.int32)
        nvis[5] = 0
        nvis[6] = 1
        nvis[70] = 33
        width = n + 5
    else:
        base = np.arange(n_q, dtype=np.int64) * n
        nvis = np.array([n - (13 * t) % 97 for t in range(n_q)], np.int32)
        nvis[3] = 0
        width = n
    qf_ref = oracle.quantize_q_mxfp4(d.q_idx)
    ref = oracle.index_score_fp4q(qf_ref, d.head_w, ix, base, nvis, width)
    for want_bm in (True, False):
        s, bm = c.index_score_fp4q(dev(qf_ref), dev(d.head_w), dev_ix(ix), dev(base), dev(nvis), width,
                                   want_block_max=want_bm)
        torch.cuda.synchronize()
        s = host(s)
        check_scores(s, ref)
        if want_bm:
            _check_bmax(s, host(bm), width)


def test_index_score_fp4q_candidate_mode(c):
    log("index_score_fp4q candidate mode")
    n_q, n, M = 3, 5000, 64
    kv, ix = synth.random_caches(19, n * n_q)
    d = synth.query_inputs(20, n_q, q_idx_scale=1.0)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.array([n, n - 3, 4001], np.int32)
    rng = np.random.default_rng(23)
    pool = np.full((n_q, M), -1, np.int32)
    for t in range(n_q):
        nb = -(-nvis[t] // 8)
        k = [M, M - 5, 17][t]
        sel = np.sort(rng.choice(nb - 1, k - 1, replace=False))
        pool[t, :k] = np.sort(np.append(sel, nb - 1))
    qf_ref = oracle.quantize_q_mxfp4(d.q_idx)
    ref = oracle.index_score_fp4q(qf_ref, d.head_w, ix, base, nvis, 8 * M, pool_blocks=pool)
    s, _ = c.index_score_fp4q(dev(qf_ref), dev(d.head_w), dev_ix(ix), dev(base), dev(nvis), 8 * M,
                              pool_blocks=dev(pool))
    torch.cuda.synchronize()
    check_scores(host(s), ref)


def test_index_score_fp4q_spread_scales(c):
    """Queries whose groups span 28 binades (E8M0 codes far from 127) through both kernels."""
    log("index_score_fp4q spread scales")
    n = 700
    kv, ix = synth.random_caches(61, n)
    rng = np.random.default_rng(62)
    for n_q in (2, 64):
        qb = _spread_q(63 + n_q, n_q)
        hw = (rng.standard_normal((n_q, 32)) / np.sqrt(32)).astype(np.float32)
        base = np.zeros(n_q, np.int64)
        nvis = np.full(n_q, n, np.int32)
        qf_ref = oracle.quantize_q_mxfp4(qb)
        ref = oracle.index_score_fp4q(qf_ref, hw, ix, base, nvis, n)
        s, _ = c.index_score_fp4q(dev(qf_ref), dev(hw), dev_ix(ix), dev(base), dev(nvis), n, want_block_max=False)
        torch.cuda.synchronize()
        check_scores(host(s), ref)


# ------------------------------------------------------------------ full-size workloads
def test_prefill_chunk4096_fp4q(c):
    """The prefill chunk's causal scoring (4096 queries x <= 34816 entries, one sequence) with
    MXFP4 queries in the bench's launch geometry, then per-query Top-512; 10 sampled queries
    through the oracle (scores and Top-512)."""
    hist_entries, chunk, m = 32768, 4096, 2
    n = hist_entries + chunk // m
    log("prefill fp4q: drawing caches")
    kv, ix = synth.random_caches(414, n)
    d = synth.query_inputs(416, chunk)
    nvis = synth.prefill_nvis(2 * hist_entries, chunk, m)
    base = np.zeros(chunk, np.int64)
    log("prefill fp4q: GPU pack + score + select")
    qf = c.quantize_q_mxfp4(bf16(d.q_idx))
    s, _ = c.index_score_fp4q(qf, dev(d.head_w), dev_ix(ix), dev(base), dev(nvis), n, want_block_max=False)
    _, topk = c.block_topk(s, dev(nvis), K=512, M=2048, want_pool=False)
    torch.cuda.synchronize()
    qf, s, topk = host(qf), host(s), host(topk)
    for t in list(range(511, chunk, 512)) + [0, 1]:
        log(f"prefill fp4q: oracle for query {t}")
        qref = oracle.quantize_q_mxfp4(d.q_idx[t:t + 1])
        assert np.array_equal(qf[t:t + 1], qref)
        s_ref = oracle.index_score_fp4q(qref, d.head_w[t:t + 1], ix, base[t:t + 1], nvis[t:t + 1], n)
        check_scores(s[t:t + 1], s_ref)
        _, tk_ref = oracle.block_topk(s_ref, nvis[t:t + 1], K=512, M=2048)
        check_selection(topk[t], tk_ref[0], lambda ids: s_ref[0, ids].astype(np.float64))


def test_decode_1m_fp4q_query(c):
    """One Full-layer decode batch at 1M context (4 x 524288 entries) with MXFP4 queries:
    scores, block maxima and Top-512 of query 2 through the oracle."""
    n, n_q = 524288, 4
    log("decode 1M fp4q: drawing caches")
    kv, ix = synth.random_caches(313, n * n_q)
    d = synth.query_inputs(314, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.full(n_q, n, np.int32)
    log("decode 1M fp4q: GPU pack + score + select")
    qf = c.quantize_q_mxfp4(bf16(d.q_idx))
    s, bm = c.index_score_fp4q(qf, dev(d.head_w), dev_ix(ix), dev(base), dev(nvis), n)
    _, topk = c.block_topk(s, dev(nvis), K=512, M=2048, block_max=bm, want_pool=False)
    torch.cuda.synchronize()
    s, bm, topk = host(s), host(bm), host(topk)
    t = 2
    log("decode 1M fp4q: oracle for query 2")
    s_ref = oracle.index_score_fp4q(oracle.quantize_q_mxfp4(d.q_idx[t:t + 1]), d.head_w[t:t + 1], ix,
                                    base[t:t + 1], nvis[t:t + 1], n)
    check_scores(s[t:t + 1], s_ref)
    _check_bmax(s[t:t + 1], bm[t:t + 1], n)
    _, tk_ref = oracle.block_topk(s_ref, nvis[t:t + 1], K=512, M=2048)
    check_selection(topk[t], tk_ref[0], lambda ids: s_ref[0, ids].astype(np.float64))
