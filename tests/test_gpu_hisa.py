"""GPU parity of HISA's coarse filter: the block-mean records bit-exact against the oracle
(ragged sequences, partial blocks, wide scale spreads so the fp32 sums round, the decode
update of the newest block alone), the pool-only selection bit-exact on identical block
scores, and the whole HISA chain (block means -> scores of the means -> pool -> scores of
the candidates -> Top-512) against the oracle's chain, at a small size and on a sampled
query of the 1M-context batch-4 decode."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth
from tests.gpu_util import bf16, check_scores, check_selection, dev, dev_ix, host, host_ix, ix_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_csa2_amd import csa2
    return csa2


def log(msg):
    print(msg, flush=True)


def _wide_caches(seed, n):
    """Indexer rows with E8M0 scales spread over 40 binades (the block sums then round) and
    a few all-zero entries."""
    _, ix = synth.random_caches(seed, n)
    rng = np.random.default_rng(seed + 1)
    ix[:, 64:] = rng.integers(100, 141, (n, 4), dtype=np.uint8)
    ix[::37, :64] = 0
    return ix


def test_block_mean_pack_bit_exact(c):
    lens = [1000, 8, 13, 1, 4096 + 5]
    log(f"block_mean_pack sequences {lens}")
    ix = _wide_caches(71, sum(lens))
    base = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    nbs = [-(-n // 8) for n in lens]
    mbase = np.concatenate([[0], np.cumsum(nbs)[:-1]]).astype(np.int64)
    ref = np.concatenate([oracle.block_mean_pack(ix[b:b + n]) for b, n in zip(base, lens)])
    out = ix_tensor(sum(nbs), 0xAB)
    c.block_mean_pack(dev_ix(ix), dev(base), dev(np.array(lens, np.int32)), max(nbs), out, dev(mbase))
    torch.cuda.synchronize()
    got = host_ix(out, sum(nbs))
    bad = np.flatnonzero(np.any(got != ref, axis=1))
    assert bad.size == 0, f"{bad.size} records differ, first {bad[:8]}"


def test_block_mean_decode_update_touches_only_the_newest_block(c):
    """After one more entry per sequence, re-packing only block (n - 1) / 8 gives the oracle's
    records for the longer sequences and leaves every other record as it was."""
    n0, n_seq = 811, 3
    ix = _wide_caches(72, n_seq * 1024)
    base = np.arange(n_seq, dtype=np.int64) * 1024
    nb_max = 1024 // 8
    mbase = np.arange(n_seq, dtype=np.int64) * nb_max
    lens = np.array([n0, n0 + 5, n0 + 13], np.int32)
    out = ix_tensor(n_seq * nb_max)
    c.block_mean_pack(dev_ix(ix), dev(base), dev(lens), nb_max, out, dev(mbase))
    before = host_ix(out).copy()
    lens2 = lens + 1
    first = ((lens2 - 1) // 8).astype(np.int32)
    c.block_mean_pack(dev_ix(ix), dev(base), dev(lens2), 1, out, dev(mbase), first_block=dev(first))
    torch.cuda.synchronize()
    after = host_ix(out)
    for s in range(n_seq):
        ref = oracle.block_mean_pack(ix[base[s]:base[s] + lens2[s]])
        rows = slice(mbase[s], mbase[s] + len(ref))
        assert np.array_equal(after[rows], ref), s
        changed = np.flatnonzero(np.any(after[mbase[s]:mbase[s] + nb_max] != before[mbase[s]:mbase[s] + nb_max], 1))
        assert set(changed.tolist()) <= {int(first[s])}, (s, changed)


@pytest.mark.parametrize("nbw,nvis,M,seed", [
    (300, [2400, 1603, 2399, 240, 0], 40, 73),
    (65536, [524288, 524281], 2048, 74),
    (2048, [16384], 2048, 75),
])
def test_pool_only_mode_bit_exact(c, nbw, nvis, M, seed):
    log(f"pool-only nbw={nbw} nvis={nvis} M={M}")
    rng = np.random.default_rng(seed)
    nvis = np.array(nvis, np.int32)
    bs = rng.standard_normal((len(nvis), nbw)).astype(np.float32)
    bs[0, ::3] = bs[0, 7]  # ties
    bs[-1, 5:50] = np.nan
    ref = oracle.pool_from_block_scores(bs, nvis, M=M)
    pool, tk = c.block_topk(None, dev(nvis), K=512, M=M, block_max=dev(bs), want_topk=False)
    torch.cuda.synchronize()
    assert tk is None
    assert np.array_equal(host(pool), ref)


def _gpu_hisa(c, d, ix_d, base, nvis, n_per_seq, M=2048, K=512):
    """GPU HISA chain for sequences of n_per_seq cache rows each (row base[t] is entry 0)."""
    n_q = len(base)
    nbw = -(-n_per_seq // 8)
    means = ix_tensor(n_q * nbw)
    mbase = np.arange(n_q, dtype=np.int64) * nbw
    c.block_mean_pack(ix_d, dev(base), dev(nvis), nbw, means, dev(mbase))
    nb_vis = ((nvis + 7) // 8).astype(np.int32)
    s_blk, _ = c.index_score(bf16(d.q_idx), dev(d.head_w), means, dev(mbase), dev(nb_vis), nbw, want_block_max=False)
    pool, _ = c.block_topk(None, dev(nvis), K=K, M=M, block_max=s_blk, want_topk=False)
    s_c, _ = c.index_score(bf16(d.q_idx), dev(d.head_w), ix_d, dev(base), dev(nvis), 8 * M, pool_blocks=pool)
    _, tk = c.block_topk(s_c, dev(nvis), K=K, pool_blocks=pool)
    torch.cuda.synchronize()
    return host_ix(means), host(s_blk), host(pool), host(s_c), host(tk)


def _oracle_check_query(t, d, ix, base, nvis, n_per_seq, got, M=2048, K=512):
    means_g, s_blk_g, pool_g, s_c_g, tk_g = got
    nbw = -(-n_per_seq // 8)
    n = int(nvis[t])
    means = oracle.block_mean_pack(ix[base[t]:base[t] + n])
    assert np.array_equal(means_g[t * nbw:t * nbw + len(means)], means), "block-mean records differ"
    nb = len(means)
    s_blk = oracle.index_score(d.q_idx[t:t + 1], d.head_w[t:t + 1], means, np.zeros(1, np.int64),
                               np.array([nb], np.int32), nbw)
    check_scores(s_blk_g[t:t + 1], s_blk)
    pool = oracle.pool_from_block_scores(s_blk, nvis[t:t + 1], M=M)
    check_selection(pool_g[t], pool[0], lambda ids: s_blk[0, ids].astype(np.float64), "hisa pool")
    # stage-wise: the oracle's token-level stage scores the GPU's pool once it has passed its check
    pool = pool_g[t:t + 1]
    s_c = oracle.index_score(d.q_idx[t:t + 1], d.head_w[t:t + 1], ix, base[t:t + 1], nvis[t:t + 1], 8 * M,
                             pool_blocks=pool)
    check_scores(s_c_g[t:t + 1], s_c)
    _, tk = oracle.block_topk(s_c, nvis[t:t + 1], K=K, pool_blocks=pool)
    pos = {int(b) * 8 + o: 8 * i + o for i, b in enumerate(pool[0]) if b >= 0 for o in range(8)}
    check_selection(tk_g[t], tk[0], lambda ids: np.array([s_c[0, pos[int(j)]] for j in ids], np.float64),
                    "hisa topk")


def test_hisa_chain_small(c):
    n, n_q, M, K = 5000, 3, 64, 64
    log("hisa chain small")
    _, ix = synth.random_caches(76, n * n_q)
    d = synth.query_inputs(77, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.array([n, n - 3, 2001], np.int32)
    got = _gpu_hisa(c, d, dev_ix(ix), base, nvis, n, M=M, K=K)
    for t in range(n_q):
        _oracle_check_query(t, d, ix, base, nvis, n, got, M=M, K=K)


def test_hisa_chain_decode_1m_b4(c):
    n, n_q = 524288, 4
    log("hisa chain 1M: drawing caches")
    _, ix = synth.random_caches(78, n * n_q)
    d = synth.query_inputs(79, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.full(n_q, n, np.int32)
    log("hisa chain 1M: GPU")
    got = _gpu_hisa(c, d, dev_ix(ix), base, nvis, n)
    log("hisa chain 1M: oracle for query 1")
    _oracle_check_query(1, d, ix, base, nvis, n, got)
