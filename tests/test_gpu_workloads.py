"""GPU parity at the full sizes of the seeded workloads, on the launch geometry the bench uses.

The GPU runs every query; the oracle recomputes sampled queries one by one from the same
inputs.  The packed caches of the long-context workloads are drawn directly (the oracle
cannot compress 10^6 entries inside a test); the prefill chunk is compressed from its
latents by both sides.  Acceptance is the one in tests/gpu_util.py."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth
from tests.gpu_util import bf16, check_attn, check_scores, check_selection, dev, dev_ix, host, host_ix

pytestmark = pytest.mark.gpu

K, M = 512, 2048


@pytest.fixture(scope="module")
def c():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_csa2_amd import csa2
    return csa2


def log(msg):
    print(msg, flush=True)


def _blockmax(row, n):
    nb = -(-n // 8)
    b = np.full(nb * 8, -np.inf)
    b[:n] = np.where(np.isnan(row[:n]), -np.inf, row[:n])
    g = b.reshape(nb, 8).max(axis=1)
    g[nb - 1] = np.inf
    return g


def _compare_query(t, s_gpu, bm_gpu, pool_gpu, topk_gpu, out_gpu, q, d, kv, ix, base, nvis, width, M=M):
    """Oracle chain for query t alone, compared with the GPU's row t, stage by stage: each
    stage's oracle consumes the GPU's output of the stage before once that output has passed
    its own check (a selection equal up to near-ties of the K-th score), so every stage is
    compared for every sampled query.  Returns the GPU's pool and Top-K rows and a dict
    counting the comparisons made."""
    seen = {"scores": 0, "pool": 0, "topk": 0, "attn": 0}
    s_ref = oracle.index_score(q.q_idx[t:t + 1], q.head_w[t:t + 1], ix, base[t:t + 1], nvis[t:t + 1], width)
    check_scores(s_gpu[t:t + 1], s_ref)
    seen["scores"] += 1
    pool_ref, topk_ref = oracle.block_topk(s_ref, nvis[t:t + 1], K=K, M=M)
    g = _blockmax(s_ref[0], nvis[t])
    if pool_gpu is not None:
        check_selection(pool_gpu[t], pool_ref[0], lambda ids: g[ids], "pool")
        seen["pool"] += 1
    check_selection(topk_gpu[t], topk_ref[0], lambda ids: s_ref[0, ids].astype(np.float64), "topk")
    seen["topk"] += 1
    if out_gpu is not None:
        o_ref, _ = oracle.sparse_attn(d.q[t:t + 1], kv, base[t:t + 1], topk_gpu[t:t + 1], d.swa,
                                      d.swa_start[t:t + 1], d.swa_len[t:t + 1])
        check_attn(out_gpu[t:t + 1], o_ref)
        seen["attn"] += 1
    return (None if pool_gpu is None else pool_gpu[t]), topk_gpu[t], seen


def test_decode_1m_b4_m2(c):
    """4 sequences x 524288 FP4 entries (1M tokens at m = 2), Full layer; queries 0 and 3 checked."""
    n, n_q = 524288, 4
    log("decode 1M: drawing caches")
    kv, ix = synth.random_caches(303, n * n_q)
    d = synth.query_inputs(304, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.full(n_q, n, np.int32)
    log("decode 1M: GPU path")
    kv_d, ix_d = dev(kv), dev_ix(ix)
    s, bm = c.index_score(bf16(d.q_idx), dev(d.head_w), ix_d, dev(base), dev(nvis), n)
    pool, topk = c.block_topk(s, dev(nvis), K=K, M=M, block_max=bm)
    out, _ = c.sparse_attn(bf16(d.q), kv_d, dev(base), topk, bf16(d.swa), dev(d.swa_start), dev(d.swa_len))
    torch.cuda.synchronize()
    s, bm, pool, topk, out = host(s), host(bm), host(pool), host(topk), host(out)
    compared = 0
    for t in (0, 3):
        log(f"decode 1M: oracle for query {t}")
        _, _, seen = _compare_query(t, s, bm, pool, topk, out, d, d, kv, ix, base, nvis, n)
        compared += seen["attn"]
    assert compared == 2, "every sampled query reaches the attention comparison"


def test_decode_1m_spread_scales(c):
    """A full-size 1M-context row (524288 entries, 2 queries) whose scale bytes cover the whole
    E4M3 range (main KV) and E8M0 codes 16 .. 240 (indexer K, 2^-111 .. 2^113), through the
    bf16-query scan, the selection and attention, both queries checked stage by stage."""
    n, n_q = 524288, 2
    log("decode 1M spread scales: drawing caches")
    kv, ix = synth.random_caches(313, n * n_q, spread_scales=True)
    d = synth.query_inputs(314, n_q)
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.full(n_q, n, np.int32)
    kv_d, ix_d = dev(kv), dev_ix(ix)
    s, bm = c.index_score(bf16(d.q_idx), dev(d.head_w), ix_d, dev(base), dev(nvis), n)
    pool, topk = c.block_topk(s, dev(nvis), K=K, M=M, block_max=bm)
    out, _ = c.sparse_attn(bf16(d.q), kv_d, dev(base), topk, bf16(d.swa), dev(d.swa_start), dev(d.swa_len))
    torch.cuda.synchronize()
    s, bm, pool, topk, out = host(s), host(bm), host(pool), host(topk), host(out)
    assert np.all(np.isfinite(s)), "scores stay finite across the spread scales"
    for t in range(n_q):
        log(f"decode 1M spread scales: oracle for query {t}")
        _, _, seen = _compare_query(t, s, bm, pool, topk, out, d, d, kv, ix, base, nvis, n)
        assert seen["attn"] == 1


def test_decode_128k_b16_full_reindex_reuse(c):
    """16 x 131072 entries at m = 1: Full (pool), Reindex (fresh N(0,1) q over the pool), 3 Reuse
    layers on the Reindex indices; sampled queries 0, 7, 15 go through the oracle."""
    n, n_q = 131072, 16
    log("128K: drawing caches")
    kv, ix = synth.random_caches(202, n * n_q)
    full = synth.query_inputs(203, n_q)
    rein = synth.query_inputs(204, n_q, q_idx_scale=1.0)
    reuse = [synth.query_inputs(205 + i, n_q) for i in range(3)]
    base = np.arange(n_q, dtype=np.int64) * n
    nvis = np.full(n_q, n, np.int32)
    kv_d, ix_d, base_d, nvis_d = dev(kv), dev_ix(ix), dev(base), dev(nvis)
    log("128K: GPU Full layer")
    s, bm = c.index_score(bf16(full.q_idx), dev(full.head_w), ix_d, base_d, nvis_d, n)
    pool, topk_f = c.block_topk(s, nvis_d, K=K, M=M, block_max=bm)
    out_f, _ = c.sparse_attn(bf16(full.q), kv_d, base_d, topk_f, bf16(full.swa), dev(full.swa_start),
                             dev(full.swa_len))
    log("128K: GPU Reindex + Reuse layers")
    s_r, _ = c.index_score(bf16(rein.q_idx), dev(rein.head_w), ix_d, base_d, nvis_d, 8 * M, pool_blocks=pool)
    _, topk_r = c.block_topk(s_r, nvis_d, K=K, pool_blocks=pool)
    out_r, _ = c.sparse_attn(bf16(rein.q), kv_d, base_d, topk_r, bf16(rein.swa), dev(rein.swa_start),
                             dev(rein.swa_len))
    outs = []
    for u in reuse:
        o, _ = c.sparse_attn(bf16(u.q), kv_d, base_d, topk_r, bf16(u.swa), dev(u.swa_start), dev(u.swa_len))
        outs.append(o)
    torch.cuda.synchronize()
    s, bm, pool_h, topk_f, out_f = host(s), host(bm), host(pool), host(topk_f), host(out_f)
    s_r, topk_r, out_r = host(s_r), host(topk_r), host(out_r)
    outs = [host(o) for o in outs]
    counts = {"full_attn": 0, "reindex_scores": 0, "reindex_topk": 0, "reindex_reuse_attn": 0}
    for t in (0, 7, 15):
        log(f"128K: oracle for query {t}")
        pool_t, _, seen = _compare_query(t, s, bm, pool_h, topk_f, out_f, full, full, kv, ix, base, nvis, n)
        counts["full_attn"] += seen["attn"]
        # the Reindex layer re-scores the GPU's pool (checked above) with its own query
        sr_ref = oracle.index_score(rein.q_idx[t:t + 1], rein.head_w[t:t + 1], ix, base[t:t + 1], nvis[t:t + 1],
                                    8 * M, pool_blocks=pool_t[None])
        check_scores(s_r[t:t + 1], sr_ref)
        counts["reindex_scores"] += 1
        _, tr_ref = oracle.block_topk(sr_ref, nvis[t:t + 1], K=K, pool_blocks=pool_t[None])
        pos = {int(b) * 8 + o: 8 * i + o for i, b in enumerate(pool_t) if b >= 0 for o in range(8)}
        check_selection(topk_r[t], tr_ref[0],
                        lambda ids: np.array([sr_ref[0, pos[int(j)]] for j in ids], np.float64), "reindex topk")
        counts["reindex_topk"] += 1
        # Reindex attention and the 3 Reuse layers attend with the GPU's (checked) Reindex Top-K
        for layer, (qin, o_gpu) in enumerate([(rein, out_r)] + list(zip(reuse, outs))):
            o_ref, _ = oracle.sparse_attn(qin.q[t:t + 1], kv, base[t:t + 1], topk_r[t:t + 1], qin.swa,
                                          qin.swa_start[t:t + 1], qin.swa_len[t:t + 1])
            check_attn(o_gpu[t:t + 1], o_ref)
            counts["reindex_reuse_attn"] += 1
    log(f"128K: comparisons {counts}")
    assert counts == {"full_attn": 3, "reindex_scores": 3, "reindex_topk": 3, "reindex_reuse_attn": 12}


def test_prefill_chunk4096_hist65536_m2(c):
    """4096-query chunk on a 65536-token history at m = 2: compress the 2048 new entries from
    their latents (bit-exact, all of them), causal scoring of 4096 x <= 34816 entries,
    per-query Top-512 and attention for all queries; 16 sampled queries go through the oracle."""
    hist_entries, chunk, m = 32768, 4096, 2
    n_new = chunk // m
    n = hist_entries + n_new
    log("prefill: drawing history caches and chunk latents")
    kv, ix = synth.random_caches(404, n)
    ci = synth.compress_inputs(405, n_new, m, first_entry=hist_entries)
    kv_new_ref, ix_new_ref = oracle.compress_pack(ci.latent, m, ci.pool_w, oracle.rope_table(ci.positions), ci.w_idx)
    kv_d, ix_d = dev(kv), dev_ix(ix)
    log("prefill: GPU compress of the chunk into the caches")
    t0 = hist_entries // 32  # the history ends at a tile boundary: the chunk's entries start a tile
    c.compress_pack(bf16(ci.latent), m, dev(ci.pool_w), dev(c.rope_table(ci.positions).numpy()), bf16(ci.w_idx),
                    kv_out=kv_d[hist_entries:], idx_out=ix_d[t0:])
    torch.cuda.synchronize()
    assert np.array_equal(host(kv_d[hist_entries:]), kv_new_ref)
    assert np.array_equal(host_ix(ix_d[t0:], n_new), ix_new_ref)
    kv[hist_entries:], ix[hist_entries:] = kv_new_ref, ix_new_ref
    nvis = synth.prefill_nvis(2 * hist_entries, chunk, m)
    d = synth.query_inputs(406, chunk, swa_rows=chunk + 127, swa_start=np.arange(chunk, dtype=np.int64),
                           swa_len=np.full(chunk, 128, np.int32))
    base = np.zeros(chunk, np.int64)
    log("prefill: GPU index + select + attention for 4096 queries")
    s, _ = c.index_score(bf16(d.q_idx), dev(d.head_w), ix_d, dev(base), dev(nvis), n, want_block_max=False)
    _, topk = c.block_topk(s, dev(nvis), K=K, M=M, want_pool=False)
    out, _ = c.sparse_attn(bf16(d.q), kv_d, dev(base), topk, bf16(d.swa), dev(d.swa_start), dev(d.swa_len))
    torch.cuda.synchronize()
    s, topk, out = host(s), host(topk), host(out)
    compared = 0
    sample = list(range(255, chunk, 256)) + [0, 1]
    for t in sample:
        log(f"prefill: oracle for query {t}")
        _, _, seen = _compare_query(t, s, None, None, topk, out, d, d, kv, ix, base, nvis, n)
        compared += seen["attn"]
    assert compared == len(sample)
