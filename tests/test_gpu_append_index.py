"""GPU parity of the fused decode append + indexer scoring (csa2_append_index_score and its
MXFP4-query twin): bit for bit what csa2_compress_append followed by csa2_index_score
produce (cache bytes, scores, block maxima), the appended bytes against the oracle's
compressor, the scores against the oracle's indexer over the updated cache, two calls in a
row, ragged rows, an empty row, rows whose newest entry opens a block or a tile, rows
shorter or longer than the score width, 70 and 300 queries at once, the MXFP4 query packed inside
the launch (special scales included), the variant that also counts the selection's first pass
(csa2_append_index_score_sel, then csa2_block_topk_prebuilt), and the 1M-context batch-4
decode in the launch geometry the bench uses.  The appended rows start out holding other bytes,
so a score computed from stale bytes would show."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth
from tests.gpu_util import bf16, check_scores, dev, dev_ix, host, host_ix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_csa2_amd import csa2
    return csa2


def log(msg):
    print(msg, flush=True)


class Case:
    """n_q sequences of rows_per_seq cache rows each, query t appending entry nvis[t] - 1."""

    def __init__(self, c, seed, nvis, width, m, rows_per_seq=None):
        self.nvis = np.array(nvis, np.int32)
        self.n_q = n_q = len(nvis)
        self.width, self.m = width, m
        self.rows = rows_per_seq or max(1, int(self.nvis.max()))
        self.kv, self.ix = synth.random_caches(seed, n_q * self.rows)
        self.base = np.arange(n_q, dtype=np.int64) * self.rows
        self.ci = synth.compress_inputs(seed + 1, n_q, m)
        self.pos = (np.maximum(self.nvis, 1) - 1).astype(np.int64) * m
        self.cs = c.rope_table(self.pos).numpy()
        self.d = synth.query_inputs(seed + 2, n_q)
        self.dst = np.where(self.nvis > 0, self.base + self.nvis - 1, -1).astype(np.int64)


def _separate(c, k, fp4):
    kv, ix = dev(k.kv), dev_ix(k.ix)
    c.compress_append(bf16(k.ci.latent), k.m, dev(k.ci.pool_w), dev(k.cs), bf16(k.ci.w_idx), dev(k.dst), kv, ix)
    q = c.quantize_q_mxfp4(bf16(k.d.q_idx)) if fp4 else bf16(k.d.q_idx)
    score = c.index_score_fp4q if fp4 else c.index_score
    s, b = score(q, dev(k.d.head_w), ix, dev(k.base), dev(k.nvis), k.width)
    return kv, ix, s, b


def _fused(c, k, fp4, kv=None, ix=None, pack_q=False):
    """fp4 with pack_q: the bf16 query goes in and the launch packs it to MXFP4 itself."""
    kv = dev(k.kv) if kv is None else kv
    ix = dev_ix(k.ix) if ix is None else ix
    q = c.quantize_q_mxfp4(bf16(k.d.q_idx)) if fp4 and not pack_q else bf16(k.d.q_idx)
    s, b = c.append_index_score(bf16(k.ci.latent), k.m, dev(k.ci.pool_w), dev(k.cs), bf16(k.ci.w_idx), kv, ix, q,
                                dev(k.d.head_w), dev(k.base), dev(k.nvis), k.width, pack_q=pack_q)
    return kv, ix, s, b


def _same(a, b):
    for x, y, what in zip(a, b, ("main-KV cache", "indexer cache", "scores", "block maxima")):
        gx, gy = host(x), host(y)
        if gx.dtype == np.float32:
            gx, gy = gx.view(np.uint32), gy.view(np.uint32)
        bad = np.argwhere(gx != gy)
        assert bad.size == 0, f"{what}: {len(bad)} elements differ, first {bad[:4].tolist()}"


CASES = [
    # nvis per query, width, m
    ([1000, 8, 9, 33, 1, 0, 4096], 4096, 2),  # blocks opened by the new entry, a lone entry, an empty row
    ([777, 32, 64, 65], 800, 1),               # rows shorter than the width, tile edges
    ([5000, 4999, 4993, 4992], 5000, 2),
    ([900, 850, 800, 799, 33], 800, 2),        # rows longer than the width: the new entry has no slot
    ([200 - (i % 9) for i in range(70)], 256, 1),  # 70 queries, one sequence each
    # 300 queries: more workgroups than fit on the device at once (several rounds)
    ([96 + (i % 31) for i in range(300)], 128, 2),
]


QFORMATS = [(False, False), (True, False), (True, True)]
QIDS = ["bf16_q", "fp4_q", "fp4_q_packed_in_launch"]


@pytest.mark.parametrize("fp4,pack_q", QFORMATS, ids=QIDS)
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_fused_equals_append_then_score(c, ci, fp4, pack_q):
    nvis, width, m = CASES[ci]
    log(f"append_index nvis={nvis} width={width} m={m} fp4={fp4} pack_q={pack_q}")
    k = Case(c, 500 + 10 * ci, nvis, width, m)
    ref = _separate(c, k, fp4)
    got = _fused(c, k, fp4, pack_q=pack_q)
    torch.cuda.synchronize()
    _same(ref, got)
    # a second call on the result appends the same entries again: same results
    again = _fused(c, k, fp4, kv=got[0], ix=got[1], pack_q=pack_q)
    torch.cuda.synchronize()
    _same(ref, again)


def _host_hist(block_max, nvis, width):
    """The selection's first-pass counts from the block maxima: per query, its older blocks
    (all but the one holding entry min(nvis, width) - 1) binned by the top 12 bits of the
    order-preserving key of their maximum (NaN ranks as -inf)."""
    bm = host(block_max).astype(np.float32)
    n_q = bm.shape[0]
    out = np.zeros((n_q, 4096), np.int64)
    for t in range(n_q):
        nw = min(int(nvis[t]), width)
        if nw <= 0:
            continue
        older = (nw - 1) // 8  # blocks 0 .. older - 1
        v = np.where(np.isnan(bm[t, :older]), -np.inf, bm[t, :older]).astype(np.float32).view(np.uint32)
        key = np.where(v & 0x80000000, ~v, v | 0x80000000).astype(np.uint32)
        out[t] = np.bincount(key >> 20, minlength=4096)
    return out


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_fused_sel_counts_and_prebuilt_selection(c, ci):
    """csa2_append_index_score_sel: the same bytes, scores and maxima as csa2_append_index_score,
    and the selection workspace's histogram rows hold exactly the first-pass counts of the
    maxima it wrote; csa2_block_topk_prebuilt on that workspace gives block_topk's pool and
    Top-K bit for bit (the short-row path included) and leaves the histogram region zero."""
    nvis, width, m = CASES[ci]
    M, K = (64, 32) if width < 4096 else (256, 128)
    log(f"append_index_sel nvis[:4]={nvis[:4]} n_q={len(nvis)} width={width} m={m} M={M} K={K}")
    k = Case(c, 600 + 10 * ci, nvis, width, m)
    ref = _fused(c, k, False)
    ws = torch.zeros(c.block_topk_workspace(k.n_q, width, M, K), dtype=torch.uint8, device="cuda")
    kv, ix = dev(k.kv), dev_ix(k.ix)
    s, b = c.append_index_score(bf16(k.ci.latent), k.m, dev(k.ci.pool_w), dev(k.cs), bf16(k.ci.w_idx), kv, ix,
                                bf16(k.d.q_idx), dev(k.d.head_w), dev(k.base), dev(k.nvis), width, sel_workspace=ws)
    torch.cuda.synchronize()
    _same(ref, (kv, ix, s, b))
    hist = host(ws[: k.n_q * 4096 * 4].view(torch.int32)).reshape(k.n_q, 4096)
    want = _host_hist(b, k.nvis, width)
    bad = np.argwhere(hist != want)
    assert bad.size == 0, f"histogram counts differ at {bad[:4].tolist()}"
    pool_ref, topk_ref = c.block_topk(ref[2], dev(k.nvis), K=K, M=M, block_max=ref[3])
    pool, topk = c.block_topk(s, dev(k.nvis), K=K, M=M, block_max=b, workspace=ws, hist_ready=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(pool), host(pool_ref)) and np.array_equal(host(topk), host(topk_ref))
    assert int(ws[: k.n_q * 4096 * 4].view(torch.int32).abs().sum().item()) == 0, "histogram region not zero"


def test_fused_sel_decode_1m_b4(c):
    """The first-pass counts at the bench's geometry (4 x 524288 entries, M = 2048, K = 512):
    exact counts, and the prebuilt selection equal to block_topk's."""
    n, n_q, M, K = 524288, 4, 2048, 512
    log("append_index_sel 1M: drawing caches")
    k = Case(c, 620, [n, n - 1, n - 8, n - 9], n, 2)
    ref = _fused(c, k, False)
    ws = torch.zeros(c.block_topk_workspace(n_q, n, M, K), dtype=torch.uint8, device="cuda")
    kv, ix = dev(k.kv), dev_ix(k.ix)
    s, b = c.append_index_score(bf16(k.ci.latent), k.m, dev(k.ci.pool_w), dev(k.cs), bf16(k.ci.w_idx), kv, ix,
                                bf16(k.d.q_idx), dev(k.d.head_w), dev(k.base), dev(k.nvis), n, sel_workspace=ws)
    torch.cuda.synchronize()
    _same(ref, (kv, ix, s, b))
    hist = host(ws[: n_q * 4096 * 4].view(torch.int32)).reshape(n_q, 4096)
    assert np.array_equal(hist, _host_hist(b, k.nvis, n)), "histogram counts differ"
    pool_ref, topk_ref = c.block_topk(ref[2], dev(k.nvis), K=K, M=M, block_max=ref[3])
    pool, topk = c.block_topk(s, dev(k.nvis), K=K, M=M, block_max=b, workspace=ws, hist_ready=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(pool), host(pool_ref)) and np.array_equal(host(topk), host(topk_ref))
    assert int(ws[: n_q * 4096 * 4].view(torch.int32).abs().sum().item()) == 0, "histogram region not zero"


def test_query_packed_in_launch_takes_every_scale_path(c):
    """Head vectors whose groups hit the packer's special scales (all zero, a huge and a tiny
    amax, values that round to a tie) give the same scores packed in the launch as packed by
    csa2_quantize_q_mxfp4 first."""
    nvis, width, m = CASES[1]
    log("append_index packed query, special scales")
    k = Case(c, 560, nvis, width, m)
    q = k.d.q_idx.copy()  # bf16 bit patterns
    q[0, 0, :32] = 0
    q[0, 1, 32:64] = synth.f32_to_bf16_bits(np.linspace(-3.0e38, 3.0e38, 32, dtype=np.float32))
    q[1, 2, 64:96] = synth.f32_to_bf16_bits(np.linspace(1e-30, 7e-30, 32, dtype=np.float32))
    q[2, 3, :] = synth.f32_to_bf16_bits((0.25 * np.arange(128) % 1.75).astype(np.float32))
    k.d = dataclasses.replace(k.d, q_idx=q)
    ref = _separate(c, k, True)
    got = _fused(c, k, True, pack_q=True)
    torch.cuda.synchronize()
    _same(ref, got)


@pytest.mark.parametrize("fp4", [False, True], ids=["bf16_q", "fp4_q"])
def test_fused_against_the_oracle(c, fp4):
    nvis, width, m = CASES[0]
    log(f"append_index vs oracle fp4={fp4}")
    k = Case(c, 530, nvis, width, m)
    kv, ix, s, b = _fused(c, k, fp4)
    torch.cuda.synchronize()
    kv, ix, s, b = host(kv), host_ix(ix), host(s), host(b)
    kv_ref, ix_ref = oracle.compress_pack(k.ci.latent, m, k.ci.pool_w, oracle.rope_table(k.pos), k.ci.w_idx)
    for t in range(k.n_q):
        r = k.dst[t]
        if r < 0:
            continue
        assert np.array_equal(kv[r], kv_ref[t]), f"query {t}: main-KV bytes"
        assert np.array_equal(ix[r], ix_ref[t]), f"query {t}: indexer bytes"
    untouched = np.setdiff1d(np.arange(len(k.kv)), k.dst[k.dst >= 0])
    assert np.array_equal(kv[untouched], k.kv[untouched]) and np.array_equal(ix[untouched], k.ix[untouched])
    if fp4:
        ref = oracle.index_score_fp4q(oracle.quantize_q_mxfp4(k.d.q_idx), k.d.head_w, ix, k.base, k.nvis, width)
    else:
        ref = oracle.index_score(k.d.q_idx, k.d.head_w, ix, k.base, k.nvis, width)
    check_scores(s, ref)
    nbw = -(-width // 8)
    pad = np.full((k.n_q, nbw * 8), -np.inf, np.float32)
    pad[:, :width] = s
    assert np.array_equal(b, pad.reshape(k.n_q, nbw, 8).max(axis=2)), "block maxima are not those of the scores"


@pytest.mark.parametrize("fp4", [False, True], ids=["bf16_q", "fp4_q"])
def test_fused_decode_1m_b4(c, fp4):
    """4 x 524288 entries, each query appending its sequence's last entry, as the bench's step."""
    n, n_q = 524288, 4
    log(f"append_index 1M: drawing caches fp4={fp4}")
    k = Case(c, 540 + fp4, [n] * n_q, n, 2)
    ref = _separate(c, k, fp4)
    log("append_index 1M: fused")
    got = _fused(c, k, fp4)
    torch.cuda.synchronize()
    _same(ref, got)
    # the newest tile of each row against the oracle (the rest is the plain scan, equal above)
    ix = host_ix(got[1])
    s = host(got[2])
    lo = n - 32
    for t in range(n_q):
        sub = ix[k.base[t] + lo:k.base[t] + n]
        q = k.d.q_idx[t:t + 1]
        if fp4:
            r = oracle.index_score_fp4q(oracle.quantize_q_mxfp4(q), k.d.head_w[t:t + 1], sub, np.zeros(1, np.int64),
                                        np.array([32], np.int32), 32)
        else:
            r = oracle.index_score(q, k.d.head_w[t:t + 1], sub, np.zeros(1, np.int64), np.array([32], np.int32), 32)
        check_scores(s[t:t + 1, lo:], r)


def test_fused_per_token_weights(c):
    """The fused append with per-token pooling weights ([n_q*2, 512]) equals the separate
    per-token compress_append + index_score, and its appended bytes equal the oracle's."""
    nvis, width, m = [1000, 8, 9, 33, 1, 4096], 4096, 2
    log("append_index per-token weights")
    k = Case(c, 560, nvis, width, m)
    w_tok = synth.softplus_weights(np.random.default_rng(561), k.n_q * m)
    kv, ix = dev(k.kv), dev_ix(k.ix)
    c.compress_append(bf16(k.ci.latent), m, dev(w_tok), dev(k.cs), bf16(k.ci.w_idx), dev(k.dst), kv, ix)
    s_ref, b_ref = c.index_score(bf16(k.d.q_idx), dev(k.d.head_w), ix, dev(k.base), dev(k.nvis), width)
    kv2, ix2 = dev(k.kv), dev_ix(k.ix)
    s, b = c.append_index_score(bf16(k.ci.latent), m, dev(w_tok), dev(k.cs), bf16(k.ci.w_idx), kv2, ix2,
                                bf16(k.d.q_idx), dev(k.d.head_w), dev(k.base), dev(k.nvis), width)
    torch.cuda.synchronize()
    assert np.array_equal(host(kv2), host(kv)) and np.array_equal(host(ix2), host(ix))
    assert np.array_equal(host(s).view(np.uint32), host(s_ref).view(np.uint32))
    assert np.array_equal(host(b).view(np.uint32), host(b_ref).view(np.uint32))
    kv_o, ix_o = oracle.compress_pack(k.ci.latent, m, w_tok, oracle.rope_table(k.pos), k.ci.w_idx)
    got_kv, got_ix = host(kv2), host_ix(ix2)
    for t in range(k.n_q):
        if k.dst[t] >= 0:
            assert np.array_equal(got_kv[k.dst[t]], kv_o[t]) and np.array_equal(got_ix[k.dst[t]], ix_o[t]), t
