"""GPU parity of the FP8 window path: the row packer (bit-exact) and the attention that
reads FP8 window rows from flat buffers or per-sequence rings (the attention tolerance of
tests/gpu_util.py), against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth
from tests.gpu_util import bf16, check_attn, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_csa2_amd import csa2
    return csa2


def log(msg):
    print(msg, flush=True)


def _rows(seed, n):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    x *= (2.0 ** rng.integers(-14, 14, size=(n, 8))).repeat(64, axis=1).astype(np.float32)
    x[rng.random((n, 512)) < 0.03] = 0.0
    return x


def _edge_rows():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    x[0, :64] = 0.0  # all-zero group
    x[1, :64] = -0.0  # negative zeros
    x[2, 64:128] = 448.0 * 2.0 ** -3  # on the grid's top
    x[2, 70] = 511.0 * 2.0 ** -3  # saturates (group max in (448 X, 512 X))
    x[3, :] = 1e-39  # subnormal fp32 / bf16 values: scale code 0
    x[3, 5] = 3e-39
    x[4, 128:192] = 2.0 ** -118  # smallest normal-scale groups
    # amax 200 gives X = 2^-1; x / X = -8.5, 17, 272, 0.53125, 400 are all exact E4M3 ties
    x[5, :448] = rng.choice([-4.25, 8.5, 136.0, 0.265625, 200.0], 448)
    x[5, ::64] = 200.0
    x[6, 3] = np.inf
    x[7, 100] = -np.inf
    x[8, 200] = np.nan
    x[9, :] = 3.0e38
    x[10, 448:] = -7.0  # RoPE tail carried verbatim
    return x


@pytest.mark.parametrize("case", ["random_1000", "random_3", "edges"])
def test_swa_pack_fp8_bit_exact(c, case):
    log(f"swa_pack_fp8 {case}")
    x = {"random_1000": lambda: _rows(1, 1000), "random_3": lambda: _rows(2, 3), "edges": _edge_rows}[case]()
    bits = synth.f32_to_bf16_bits(x)
    ref = oracle.swa_fp8_pack(bits)
    got = host(c.swa_pack_fp8(bf16(bits)))
    torch.cuda.synchronize()
    bad = np.any(got != ref, axis=1)
    assert not bad.any(), f"rows differ: {np.nonzero(bad)[0][:8]}"


def test_swa_pack_fp8_into_ring_slots(c):
    log("swa_pack_fp8 scatter into ring slots")
    bits = synth.f32_to_bf16_bits(_rows(3, 50))
    ref = oracle.swa_fp8_pack(bits)
    rng = np.random.default_rng(3)
    dst = rng.permutation(256)[:50].astype(np.int64)
    dst[::7] = -1  # skipped rows
    buf = torch.full((256, 584), 0xAB, dtype=torch.uint8, device="cuda")
    c.swa_pack_fp8(bf16(bits), out=buf, dst_rows=dev(dst))
    got = host(buf)
    for r in range(50):
        if dst[r] >= 0:
            assert np.array_equal(got[dst[r]], ref[r]), f"row {r} -> slot {dst[r]}"
    untouched = np.setdiff1d(np.arange(256), dst[dst >= 0])
    assert np.all(got[untouched] == 0xAB)


def _attn_case(seed, n_q, K, n_entries, ring):
    kv, _ = synth.random_caches(seed, n_entries)
    rng = np.random.default_rng(seed)
    swa_len = rng.integers(0, 129, n_q).astype(np.int32)
    swa_len[0] = 128
    rows = (ring if ring else 128) * n_q
    d = synth.query_inputs(seed + 1, n_q, swa_rows=rows, swa_len=swa_len)
    if ring:  # each sequence owns one ring; windows start anywhere in it and wrap
        start = np.arange(n_q, dtype=np.int64) * ring + rng.integers(0, ring, n_q)
    else:
        start = d.swa_start
    topk = np.full((n_q, K), -1, np.int32)
    for t in range(n_q):
        k = K if t % 3 == 0 else int(rng.integers(0, K + 1))
        topk[t, :k] = np.sort(rng.choice(n_entries, k, replace=False))
    if n_q > 1:
        topk[1] = -1  # window only
    return kv, d, start, topk


@pytest.mark.parametrize("n_q,K,n_entries,ring,seed", [(1, 512, 4096, 0, 50), (4, 512, 3000, 128, 51),
                                                        (3, 100, 500, 160, 52), (600, 512, 2048, 128, 53),
                                                        (16, 512, 2048, 0, 54)])
def test_sparse_attn_swa_fp8(c, n_q, K, n_entries, ring, seed):
    log(f"sparse_attn_swa_fp8 n_q={n_q} K={K} ring={ring}")
    kv, d, start, topk = _attn_case(seed, n_q, K, n_entries, ring)
    swa8 = oracle.swa_fp8_pack(d.swa)
    base = np.zeros(n_q, np.int64)
    ref, lse_ref = oracle.sparse_attn_swa_fp8(d.q, kv, base, topk, swa8, start, d.swa_len, swa_ring=ring)
    out, lse = c.sparse_attn_swa_fp8(bf16(d.q), dev(kv), dev(base), dev(topk), dev(swa8), dev(start),
                                     dev(d.swa_len), swa_ring=ring)
    torch.cuda.synchronize()
    rel = check_attn(host(out), ref)
    log(f"  max rel err {rel:.2e}")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(host(lse)))
    assert np.allclose(host(lse)[fin], lse_ref[fin], atol=2e-3)


def test_sparse_attn_swa_fp8_matches_bf16_window_of_dequantised_rows(c):
    """The FP8 entry point equals the bf16 entry point fed the dequantised rows."""
    log("sparse_attn_swa_fp8 vs bf16 window of dequantised rows")
    kv, d, start, topk = _attn_case(55, 8, 512, 2048, 0)
    swa8 = oracle.swa_fp8_pack(d.swa)
    deq = synth.f32_to_bf16_bits(oracle.dequant_swa_fp8(swa8).astype(np.float32))  # exact
    base = np.zeros(8, np.int64)
    o8, l8 = c.sparse_attn_swa_fp8(bf16(d.q), dev(kv), dev(base), dev(topk), dev(swa8), dev(start),
                                   dev(d.swa_len))
    ob, lb = c.sparse_attn(bf16(d.q), dev(kv), dev(base), dev(topk), bf16(deq), dev(start), dev(d.swa_len))
    torch.cuda.synchronize()
    log(f"  bit-identical: {torch.equal(o8, ob) and torch.equal(l8, lb)}")
    assert torch.allclose(o8, ob, rtol=1e-6, atol=1e-7) and torch.allclose(l8, lb, rtol=1e-6, atol=1e-7)


def test_decode_1m_b4_fp8_window_rings(c):
    """The 1M-token batch-4 decode geometry: 4 sequences x 524288 FP4 entries, each with a
    128-row FP8 window ring into which the step's new token was just packed."""
    n, n_q, ring = 524288, 4, 128
    rng = np.random.default_rng(60)
    log("decode 1M fp8 window: selected entries")
    topk = np.stack([np.sort(rng.choice(n, 512, replace=False)) for _ in range(n_q)]).astype(np.int32)
    kv_sel, _ = synth.random_caches(61, n_q * 512)  # the only entries the attention reads
    kv_d = torch.zeros((n * n_q, 288), dtype=torch.uint8, device="cuda")
    rows = (np.arange(n_q)[:, None] * n + topk).reshape(-1)
    kv_d[dev(rows.astype(np.int64))] = dev(kv_sel)
    d = synth.query_inputs(62, n_q, swa_rows=ring * n_q)
    pos = rng.integers(10 ** 6, 2 * 10 ** 6, n_q)  # newest token position of each sequence
    slot = np.arange(n_q) * ring + pos % ring
    ring_d = torch.zeros((ring * n_q, 584), dtype=torch.uint8, device="cuda")
    older = np.setdiff1d(np.arange(ring * n_q), slot)
    c.swa_pack_fp8(bf16(d.swa[older]), out=ring_d, dst_rows=dev(older.astype(np.int64)))
    c.swa_pack_fp8(bf16(d.swa[slot]), out=ring_d, dst_rows=dev(slot.astype(np.int64)))  # the step's append
    start = (np.arange(n_q) * ring + (pos + 1) % ring).astype(np.int64)  # oldest row of each window
    length = np.full(n_q, 128, np.int32)
    base = np.arange(n_q, dtype=np.int64) * n
    out, lse = c.sparse_attn_swa_fp8(bf16(d.q), kv_d, dev(base), dev(topk), ring_d, dev(start), dev(length),
                                     swa_ring=ring)
    torch.cuda.synchronize()
    swa8 = oracle.swa_fp8_pack(d.swa)
    assert np.array_equal(host(ring_d), swa8)
    for t in range(n_q):
        log(f"decode 1M fp8 window: oracle for query {t}")
        compact = np.arange(512, dtype=np.int32)[None]
        ref, lse_ref = oracle.sparse_attn_swa_fp8(d.q[t:t + 1], kv_sel[512 * t:512 * (t + 1)], [0], compact, swa8,
                                                  start[t:t + 1], length[t:t + 1], swa_ring=ring)
        check_attn(host(out[t:t + 1]), ref)
        assert np.allclose(host(lse[t:t + 1]), lse_ref, atol=2e-3)
