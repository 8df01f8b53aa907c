"""Pins for the oracle's MXFP4 indexer query (CPU only): the E8M0 scale rule against
numpy's frexp, every element against a brute-force nearest search over the E2M1 grid
(ties to the even code, saturation), exact round trips, the byte layout read back by the
already-pinned indexer-K dequantiser, and the FP4-query score equal to the bf16-query
score of the dequantised query."""
import numpy as np
import pytest

import oracle
from fp4_kv_cache_csa2_amd import synth

GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


def _q(seed, n_q=3, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_q, 32, 128)).astype(np.float32) / np.float32(np.sqrt(128.0))
    if spread:
        x *= (2.0 ** rng.integers(-20, 8, size=(n_q, 32, 4))).repeat(32, axis=2).astype(np.float32)
        x[0, 0, :32] = 0.0
        x[0, 1, 40] = 0.0
    return synth.f32_to_bf16_bits(x)


def _nearest(v, X):
    """E2M1 code (sign bit 8) of v on the grid g*X: nearest, ties to the even code, 6X cap."""
    a = abs(v)
    d = np.abs(GRID * X - a)
    best = np.flatnonzero(d == d.min())
    c = best[0] if len(best) == 1 else best[best % 2 == 0][0]
    if a >= 6 * X:
        c = 7
    return int(c | 8) if (v < 0 and c != 0) else int(c)


def test_scales_follow_the_mx_rule():
    qb = _q(1)
    out = oracle.quantize_q_mxfp4(qb)
    x = synth.bf16_bits_to_f32(qb).astype(np.float64)
    for t in range(x.shape[0]):
        for h in range(32):
            for g in range(4):
                amax = np.max(np.abs(x[t, h, 32 * g:32 * g + 32]))
                if amax == 0:
                    want = 0
                else:
                    _, e = np.frexp(np.float32(amax))
                    want = int(np.clip(e - 1 - 2 + 127, 0, 254))
                assert out[t, h, 64 + g] == want


def test_elements_are_nearest_grid_points():
    qb = _q(2, n_q=1)
    out = oracle.quantize_q_mxfp4(qb)
    x = synth.bf16_bits_to_f32(qb).astype(np.float64)
    for h in range(32):
        for ch in range(128):
            X = 2.0 ** (int(out[0, h, 64 + ch // 32]) - 127)
            code = (out[0, h, ch // 2] >> (4 * (ch & 1))) & 15
            assert code == _nearest(x[0, h, ch], X), (h, ch)


def test_round_trip_and_layout_match_the_indexer_k_format():
    rng = np.random.default_rng(3)
    n_q = 2
    codes = rng.integers(0, 16, size=(n_q, 32, 128))
    codes[codes == 8] = 0  # no negative zero in a packed vector
    s = rng.integers(100, 140, size=(n_q, 32, 4))
    for g in range(4):  # a magnitude of 4 or 6 in every group fixes the scale
        codes[:, :, 32 * g] = rng.choice([6, 7, 14, 15], size=(n_q, 32))
    vals = np.where(codes & 8, -1, 1) * GRID[codes & 7] * np.repeat(2.0 ** (s - 127), 32, axis=2)
    qb = synth.f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(qb), vals)
    out = oracle.quantize_q_mxfp4(qb)
    deq = oracle.dequant_idx(out.reshape(-1, 68)).reshape(n_q, 32, 128)  # the pinned K dequantiser
    assert np.array_equal(deq, vals)
    assert np.array_equal(out[:, :, 64:], s)


def test_fp4_query_score_equals_bf16_score_of_dequantised_query():
    kv, ix = synth.random_caches(5, 700)
    d = synth.query_inputs(6, 3)
    q4 = oracle.quantize_q_mxfp4(d.q_idx)
    qdeq = synth.f32_to_bf16_bits(oracle.dequant_idx(q4.reshape(-1, 68)).reshape(3, 32, 128).astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(qdeq).astype(np.float64),
                          oracle.dequant_idx(q4.reshape(-1, 68)).reshape(3, 32, 128))
    base = np.array([0, 100, 200], np.int64)
    nvis = np.array([500, 433, 9], np.int32)
    s4 = oracle.index_score_fp4q(q4, d.head_w, ix, base, nvis, 512)
    sb = oracle.index_score(qdeq, d.head_w, ix, base, nvis, 512)
    assert np.array_equal(s4, sb)
    pool = np.full((3, 8), -1, np.int32)
    pool[:, :5] = [[0, 3, 7, 9, 60], [1, 2, 5, 50, 53], [0, 1, -1, -1, -1]]
    assert np.array_equal(oracle.index_score_fp4q(q4, d.head_w, ix, base, nvis, 64, pool_blocks=pool),
                          oracle.index_score(qdeq, d.head_w, ix, base, nvis, 64, pool_blocks=pool))


def test_group_holding_an_infinity_takes_the_largest_finite_scale():
    """floor(log2 amax) has no value for amax = inf: such a group takes E8M0 code 254 (the
    largest finite scale, as the FP8 window rows do) and the infinite element saturates to
    the largest E2M1 magnitude; finite elements are coded against X = 2^127."""
    x = np.zeros((1, 32, 128), np.float32)
    x[0, 0, :32] = 1.0
    x[0, 0, 3] = np.inf
    x[0, 1, 32:64] = -2.0 ** 126
    x[0, 1, 40] = -np.inf
    out = oracle.quantize_q_mxfp4(synth.f32_to_bf16_bits(x))
    assert out[0, 0, 64] == 254 and out[0, 1, 65] == 254
    assert (out[0, 0, 1] >> 4) & 15 == 7                 # channel 3: +inf -> +6X
    assert out[0, 1, 20] & 15 == 15                       # channel 40: -inf -> -6X
    # -2^126 = -0.5 X: the E2M1 midpoint between 0 and 0.5 X is 0.25 X, so code 1 (0.5) with the sign
    assert (out[0, 1, 16] & 15) == 9
    # 1.0 = 2^-127 X rounds to zero
    assert out[0, 0, 0] == 0
