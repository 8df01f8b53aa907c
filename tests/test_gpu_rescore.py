"""GPU parity of the decode selection without a score row: csa2_append_index_score with
scores = NULL writes the block maxima alone, and csa2_block_topk_rescore re-scores the
candidate entries from the indexer cache.  Its pool and Top-K must equal, bit for bit,
csa2_block_topk over the score row the scan writes (and, through it, the oracle's selection
over that row): ragged rows, rows shorter or longer than the width, an empty row, spread
E8M0 scales, a tie-heavy row whose list of candidate entries is longer than the finalize's
LDS list (the selection then reads the list from global memory), the fused scan in both
modes, and the 1M-context batch-4 decode in the bench's launch geometry."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth
from tests.gpu_util import bf16, dev, dev_ix, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_csa2_amd import csa2
    return csa2


def log(msg):
    print(msg, flush=True)


def _both_paths(c, d, ix_d, base_d, nvis_d, width, K=512, M=2048, n_q=None):
    """(pool, topk) from block_topk over the GPU's score row and from block_topk_rescore over
    its block maxima, plus the score row (host)."""
    q = bf16(d.q_idx) if n_q is None else bf16(d.q_idx[:n_q])
    hw = dev(d.head_w) if n_q is None else dev(d.head_w[:n_q])
    s, bm = c.index_score(q, hw, ix_d, base_d, nvis_d, width)
    pool, topk = c.block_topk(s, nvis_d, K=K, M=M, block_max=bm)
    pool_r, topk_r = c.block_topk_rescore(bm, nvis_d, q, hw, ix_d, base_d, width, K=K, M=M)
    torch.cuda.synchronize()
    return host(pool), host(topk), host(pool_r), host(topk_r), host(s)


@pytest.mark.parametrize("n_q,n,width_pad,seed,spread", [(1, 2048, 0, 1, False), (4, 50000, 13, 2, False),
                                                         (3, 20000, 0, 3, True), (8, 9000, 777, 4, False),
                                                         (2, 100, 0, 5, False)])
def test_rescore_equals_score_row_selection(c, n_q, n, width_pad, seed, spread):
    log(f"rescore n_q={n_q} n={n} pad={width_pad} spread={spread}")
    kv, ix = synth.random_caches(seed, n * n_q, spread_scales=spread)
    d = synth.query_inputs(seed + 50, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.array([n - (977 * t) % max(n // 2, 1) for t in range(n_q)], np.int32)
    if n_q > 2:
        nvis[2] = 0  # an empty row
    width = n + width_pad
    pool, topk, pool_r, topk_r, s = _both_paths(c, d, dev_ix(ix), dev(base), dev(nvis), width)
    assert np.array_equal(pool_r, pool) and np.array_equal(topk_r, topk)
    # and the oracle's selection over the same score row
    pool_o, topk_o = oracle.block_topk(s, nvis, K=512, M=2048)
    assert np.array_equal(pool_r, pool_o) and np.array_equal(topk_r, topk_o)


def test_rescore_tie_heavy_row_beyond_the_lds_list(c):
    """Every indexer row of the sequence is one of three rows, so nearly every block ties at
    the top: the candidate list (tens of thousands of entries) is longer than the finalize's
    LDS list, the selection reads it from the global segments, and ties go to the lower index."""
    n_q, n = 2, 120000
    kv, ix = synth.random_caches(11, 3 * n_q)
    rng = np.random.default_rng(12)
    pick = rng.integers(0, 3, n * n_q)
    ix_full = ix[pick]
    d = synth.query_inputs(13, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.array([n, n - 5], np.int32)
    pool, topk, pool_r, topk_r, s = _both_paths(c, d, dev_ix(ix_full), dev(base), dev(nvis), n)
    assert np.array_equal(pool_r, pool) and np.array_equal(topk_r, topk)
    pool_o, topk_o = oracle.block_topk(s, nvis, K=512, M=2048)
    assert np.array_equal(topk_r, topk_o) and np.array_equal(pool_r, pool_o)
    # the tie structure did what it was meant to: more than 12288 candidate entries
    nb = (nvis[0] + 7) // 8
    bm = np.max(np.pad(s[0, :nvis[0]], (0, nb * 8 - nvis[0]), constant_values=-np.inf).reshape(nb, 8), axis=1)
    assert np.sum(bm[:-1] >= np.sort(bm[:-1])[-512]) * 8 > 12288


def test_many_query_scores_equal_decode_kernel_scores(c):
    """The many-query kernel (64 queries or more in one call) and the per-query decode kernel
    give the same bits, so block_topk_rescore matches the selection over either's row."""
    n_q, n = 72, 3001
    kv, ix = synth.random_caches(21, n)
    d = synth.query_inputs(22, n_q)
    base = np.zeros(n_q, np.int64)
    nvis = np.array([n - 37 * t for t in range(n_q)], np.int32)
    s_all, bm_all = c.index_score(bf16(d.q_idx), dev(d.head_w), dev_ix(ix), dev(base), dev(nvis), n)
    parts = []
    for t0 in range(0, n_q, 24):
        sl = slice(t0, t0 + 24)
        s_p, _ = c.index_score(bf16(d.q_idx[sl]), dev(d.head_w[sl]), dev_ix(ix), dev(base[sl]), dev(nvis[sl]), n)
        parts.append(host(s_p))
    torch.cuda.synchronize()
    assert np.array_equal(host(s_all).view(np.uint32), np.concatenate(parts).view(np.uint32))


@pytest.mark.parametrize("m", [1, 2])
def test_fused_scan_maxima_only_then_rescore(c, m):
    """The fused append + scan with no score row writes the same cache bytes and block maxima
    as with one, and the re-scoring selection over them equals block_topk over that row."""
    n_q, rows = 4, 30000
    rng = np.random.default_rng(31 + m)
    kv, ix = synth.random_caches(32 + m, rows * n_q)
    d = synth.query_inputs(34 + m, n_q)
    ci = synth.compress_inputs(35 + m, n_q, m)  # each query's newest entry: m latents
    base = np.arange(n_q, dtype=np.int64) * rows
    nvis = np.array([rows - int(rng.integers(0, 5000)) for _ in range(n_q)], np.int32)
    width = rows
    pos = (nvis.astype(np.int64) - 1) * m
    cs = dev(c.rope_table(pos).numpy())
    outs = []
    for want_scores in (True, False):
        kv_d, ix_d = dev(kv), dev_ix(ix)
        s, bm = c.append_index_score(bf16(ci.latent), m, dev(ci.pool_w), cs, bf16(ci.w_idx), kv_d, ix_d,
                                     bf16(d.q_idx), dev(d.head_w), dev(base), dev(nvis), width,
                                     want_scores=want_scores)
        if want_scores:
            pool, topk = c.block_topk(s, dev(nvis), block_max=bm)
        else:
            assert s is None
            pool, topk = c.block_topk_rescore(bm, dev(nvis), bf16(d.q_idx), dev(d.head_w), ix_d, dev(base), width)
        torch.cuda.synchronize()
        outs.append([host(x) for x in (kv_d, ix_d, bm, pool, topk)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_rescore_decode_1m_batch4(c):
    """The bench's workload: 4 sequences of 524288 entries, the fused scan without scores, then
    the re-scoring selection, against block_topk over the score row of the scan with scores."""
    from bench import Decode1M
    D = Decode1M(torch, c, 1 << 20, n_seq=4, m=2, ncopy=1)
    cp = D.copies[0]
    args = (cp["last_lat"].view(D.n_seq * D.m, 512), D.m, cp["pool_w"], D.cs_new[0], cp["w_idx"], cp["kv"], cp["ix"],
            cp["q_idx"], cp["head_w"], D.q_base, D.q_nvis, D.n)
    s, bm_ref = c.append_index_score(*args)  # appends and writes the score row and the maxima
    pool, topk = c.block_topk(s, D.q_nvis, block_max=bm_ref)
    s2, bm2 = c.append_index_score(*args, want_scores=False)
    pool_r, topk_r = c.block_topk_rescore(bm2, D.q_nvis, cp["q_idx"], cp["head_w"], cp["ix"], D.q_base, D.n)
    torch.cuda.synchronize()
    assert s2 is None
    assert torch.equal(bm2, bm_ref)
    assert torch.equal(pool_r, pool) and torch.equal(topk_r, topk)
