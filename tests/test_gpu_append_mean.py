"""GPU parity of HISA's fused decode step (csa2_append_mean_index_score and its MXFP4-query
twin): bit for bit what csa2_compress_append, csa2_block_mean_pack of the newest block and
csa2_index_score over the block means produce (cache bytes, block-mean records, scores,
block maxima), the new record and the scores against the oracle, two calls in a row,
ragged rows, an empty row, new entries that open a block or a tile of block means, score
widths shorter than the visible means, 70 queries at once, and the 1M-context batch-4
decode in the bench's launch geometry.  Every cache and mean row starts out holding other
bytes, so a result computed from stale bytes would show."""
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
    """n_q sequences of `rows` cache rows and rows / 8 mean rows each; query t appends entry
    nvis[t] - 1 of its sequence."""

    def __init__(self, c, seed, nvis, width, m):
        self.nvis = np.array(nvis, np.int32)
        self.n_q = n_q = len(nvis)
        self.width, self.m = width, m
        self.rows = -(-max(1, int(self.nvis.max())) // 8) * 8
        self.nbr = self.rows // 8
        self.kv, self.ix = synth.random_caches(seed, n_q * self.rows)
        _, self.means = synth.random_caches(seed + 3, n_q * self.nbr)
        self.base = np.arange(n_q, dtype=np.int64) * self.rows
        self.mbase = np.arange(n_q, dtype=np.int64) * self.nbr
        self.ci = synth.compress_inputs(seed + 1, n_q, m)
        self.pos = (np.maximum(self.nvis, 1) - 1).astype(np.int64) * m
        self.cs = c.rope_table(self.pos).numpy()
        self.d = synth.query_inputs(seed + 2, n_q)
        self.dst = np.where(self.nvis > 0, self.base + self.nvis - 1, -1).astype(np.int64)
        self.newest = np.where(self.nvis > 0, (self.nvis - 1) // 8, 0).astype(np.int32)
        self.nb = ((self.nvis.astype(np.int64) + 7) // 8).astype(np.int32)


def _q(c, k, fp4):
    return c.quantize_q_mxfp4(bf16(k.d.q_idx)) if fp4 else bf16(k.d.q_idx)


def _separate(c, k, fp4, want_bmax):
    kv, ix, mc = dev(k.kv), dev_ix(k.ix), dev_ix(k.means)
    c.compress_append(bf16(k.ci.latent), k.m, dev(k.ci.pool_w), dev(k.cs), bf16(k.ci.w_idx), dev(k.dst), kv, ix)
    c.block_mean_pack(ix, dev(k.base), dev(k.nvis), 1, mc, dev(k.mbase), first_block=dev(k.newest))
    score = c.index_score_fp4q if fp4 else c.index_score
    s, b = score(_q(c, k, fp4), dev(k.d.head_w), mc, dev(k.mbase), dev(k.nb), k.width, want_block_max=want_bmax)
    return kv, ix, mc, s, b


def _fused(c, k, fp4, want_bmax, state=None):
    kv, ix, mc = (dev(k.kv), dev_ix(k.ix), dev_ix(k.means)) if state is None else state
    s, b = c.append_mean_index_score(bf16(k.ci.latent), k.m, dev(k.ci.pool_w), dev(k.cs), bf16(k.ci.w_idx), kv, ix,
                                     mc, dev(k.mbase), _q(c, k, fp4), dev(k.d.head_w), dev(k.base), dev(k.nvis),
                                     k.width, want_block_max=want_bmax)
    return kv, ix, mc, s, b


def _same(a, b):
    for x, y, what in zip(a, b, ("main-KV cache", "indexer cache", "block means", "scores", "block maxima")):
        if x is None or y is None:
            assert x is None and y is None, what
            continue
        gx, gy = host(x), host(y)
        if gx.dtype == np.float32:
            gx, gy = gx.view(np.uint32), gy.view(np.uint32)
        bad = np.argwhere(gx != gy)
        assert bad.size == 0, f"{what}: {len(bad)} elements differ, first {bad[:4].tolist()}"


CASES = [
    # nvis per query, width (block means scored), m
    ([1000, 8, 9, 33, 1, 0, 4096], 512, 2),   # blocks opened by the new entry, a lone entry, an empty row
    ([256, 257, 255, 264, 2048], 300, 1),      # the newest mean at a tile edge (slots 31 and 32)
    ([900, 850, 800, 257], 100, 2),            # more visible means than the width: no newest slot scored
    ([1600 - 3 * (i % 11) for i in range(70)], 200, 1),  # 70 queries
    # 300 queries: more workgroups than fit on the device at once (several rounds)
    ([400 - (i % 13) for i in range(300)], 64, 2),
]


@pytest.mark.parametrize("fp4", [False, True], ids=["bf16_q", "fp4_q"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_fused_equals_append_mean_then_score(c, ci, fp4):
    nvis, width, m = CASES[ci]
    want_bmax = ci % 2 == 0
    log(f"append_mean_index nvis={nvis} width={width} m={m} fp4={fp4} block_max={want_bmax}")
    k = Case(c, 600 + 10 * ci, nvis, width, m)
    ref = _separate(c, k, fp4, want_bmax)
    got = _fused(c, k, fp4, want_bmax)
    torch.cuda.synchronize()
    _same(ref, got)
    # a second call on the result appends the same entries and re-packs the same records again
    again = _fused(c, k, fp4, want_bmax, state=got[:3])
    torch.cuda.synchronize()
    _same(ref, again)


@pytest.mark.parametrize("fp4", [False, True], ids=["bf16_q", "fp4_q"])
def test_fused_against_the_oracle(c, fp4):
    nvis, width, m = CASES[0]
    log(f"append_mean_index vs oracle fp4={fp4}")
    k = Case(c, 640, nvis, width, m)
    kv, ix, mc, s, b = _fused(c, k, fp4, True)
    kv, ix, mc, s, b = host(kv), host_ix(ix), host_ix(mc), host(s), host(b)
    kv_ref, ix_ref = oracle.compress_pack(k.ci.latent, m, k.ci.pool_w, oracle.rope_table(k.pos), k.ci.w_idx)
    touched = []
    for t in range(k.n_q):
        if k.dst[t] < 0:
            continue
        assert np.array_equal(kv[k.dst[t]], kv_ref[t]) and np.array_equal(ix[k.dst[t]], ix_ref[t]), t
        # the newest block's record: the oracle's mean of that block's entries as now cached
        lo = k.base[t] + 8 * k.newest[t]
        rec = oracle.block_mean_pack(ix[lo:k.base[t] + k.nvis[t]])
        assert len(rec) == 1 and np.array_equal(mc[k.mbase[t] + k.newest[t]], rec[0]), f"query {t}: mean record"
        touched.append(k.mbase[t] + k.newest[t])
    rest = np.setdiff1d(np.arange(len(k.means)), touched)
    assert np.array_equal(mc[rest], k.means[rest]), "a mean record other than the newest changed"
    if fp4:
        ref = oracle.index_score_fp4q(oracle.quantize_q_mxfp4(k.d.q_idx), k.d.head_w, mc, k.mbase, k.nb, width)
    else:
        ref = oracle.index_score(k.d.q_idx, k.d.head_w, mc, k.mbase, k.nb, width)
    check_scores(s, ref)
    nbw = -(-width // 8)
    pad = np.full((k.n_q, nbw * 8), -np.inf, np.float32)
    pad[:, :width] = s
    assert np.array_equal(b, pad.reshape(k.n_q, nbw, 8).max(axis=2)), "block maxima are not those of the scores"


def test_fused_decode_1m_b4(c):
    """4 x 524288 entries and 65536 block means each, the HISA step of the bench."""
    n, n_q = 524288, 4
    log("append_mean_index 1M: drawing caches")
    k = Case(c, 650, [n] * n_q, n // 8, 2)
    ref = _separate(c, k, False, False)
    log("append_mean_index 1M: fused")
    got = _fused(c, k, False, False)
    torch.cuda.synchronize()
    _same(ref, got)
    mc, s = host_ix(got[2]), host(got[3])
    nb = n // 8
    for t in range(n_q):  # the tile of block means holding the new record against the oracle
        sub = mc[k.mbase[t] + nb - 32:k.mbase[t] + nb]
        r = oracle.index_score(k.d.q_idx[t:t + 1], k.d.head_w[t:t + 1], sub, np.zeros(1, np.int64),
                               np.array([32], np.int32), 32)
        check_scores(s[t:t + 1, nb - 32:], r)
