"""GPU check of the allocation-free selection call, csa2_block_topk_noalloc, called through
the C ABI: its outputs equal csa2_block_topk's (caller's workspace) bit for bit on calls in a
row -- a 1M-context batch, then a smaller one, then a larger one (its histogram region must
be cleared again) -- in Full, candidate and pool-only modes; a problem larger than the fixed
array is rejected on the host with CSA2_ERR_SCRATCH."""
import ctypes

import numpy as np
import pytest
import torch

from fp4_kv_cache_csa2_amd import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_csa2_amd import csa2
    return csa2


def log(msg):
    print(msg, flush=True)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(c, scores, bmax, nvis, pool_blocks, M, K, pool_out, topk_out):
    n_q = nvis.numel()
    width = scores.shape[1] if scores is not None else 8 * bmax.shape[1]
    st = c._L.csa2_block_topk_noalloc(_p(scores), _p(bmax), n_q, width, _p(nvis), _p(pool_blocks), 8, M, K,
                                      _p(pool_out), _p(topk_out),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, c._L.csa2_status_string(st)


def _same(a, b, what):
    assert np.array_equal(host(a), host(b)), what


def test_noalloc_equals_workspace_call(c):
    K, M = 512, 2048
    cases = [(4, 524288, 70, 0.0), (2, 40000, 71, 0.05), (16, 131072, 72, 0.0)]  # shrink, then grow
    for n_q, width, seed, tie in cases:
        log(f"noalloc Full mode n_q={n_q} width={width}")
        s = dev(synth.random_scores(seed, n_q, width, tie_frac=tie))
        nvis = dev(np.array([width - (37 * t) % 1000 for t in range(n_q)], np.int32))
        pool_r, topk_r = c.block_topk(s, nvis, K=K, M=M)
        pool = torch.full((n_q, M), -7, dtype=torch.int32, device="cuda")
        topk = torch.full((n_q, K), -7, dtype=torch.int32, device="cuda")
        _noalloc(c, s, None, nvis, None, M, K, pool, topk)
        torch.cuda.synchronize()
        _same(pool, pool_r, "pool")
        _same(topk, topk_r, "topk")
    log("noalloc candidate and pool-only modes")
    for n_q in (8, 3):
        s = dev(synth.random_scores(80 + n_q, n_q, 8 * M))
        nvis = dev(np.full(n_q, 500000, np.int32))
        blocks = np.stack([np.sort(np.random.default_rng(t).choice(62500, M, replace=False)) for t in range(n_q)])
        blocks[:, -5:] = -1
        pb = dev(blocks.astype(np.int32))
        _, topk_r = c.block_topk(s, nvis, K=K, pool_blocks=pb)
        topk = torch.empty((n_q, K), dtype=torch.int32, device="cuda")
        _noalloc(c, s, None, nvis, pb, M, K, None, topk)
        bs = dev(synth.random_scores(90 + n_q, n_q, 62500))
        pool_r, _ = c.block_topk(None, nvis, K=K, M=M, block_max=bs, want_topk=False)
        pool = torch.empty((n_q, M), dtype=torch.int32, device="cuda")
        _noalloc(c, None, bs, nvis, None, M, K, pool, None)
        torch.cuda.synchronize()
        _same(topk, topk_r, "candidate topk")
        _same(pool, pool_r, "pool-only pool")
    # too large for the fixed array: rejected before any launch
    n_q, width = 4096, 34816
    s = torch.empty((n_q, width), dtype=torch.float32, device="cuda")
    nvis = torch.full((n_q,), width, dtype=torch.int32, device="cuda")
    topk = torch.empty((n_q, K), dtype=torch.int32, device="cuda")
    st = c._L.csa2_block_topk_noalloc(_p(s), None, n_q, width, _p(nvis), None, 8, M, K, None, _p(topk), None)
    assert st == c.ERR_SCRATCH
