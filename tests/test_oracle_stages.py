"""Pins for the oracle's four stages (CPU only).

Each pin is a fact fixed by the pages or by mathematics, not a retyping of the oracle:
equal-weight pooling is the mean, m = 1 is the identity, RoPE at position 0 is the
identity and preserves the norm, the pool that covers every block makes the
hierarchical Top-K the brute-force Top-K (numpy's sort), attention with q = 0 is the
mean of the keys, a single key is returned as is, outputs stay in the keys' convex
hull, a common shift of every logit changes nothing, and so on."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth

RNG = np.random.default_rng(1234)


def rope_id_table(n):
    t = np.zeros((n, 64), np.float32)
    t[:, :32] = 1.0
    return t


# ------------------------------------------------------------------ stage 1: compressor
def _compress(n, m, seed=0, pool_w=None, table=None):
    ci = synth.compress_inputs(seed, n, m)
    pw = ci.pool_w if pool_w is None else pool_w
    cs = oracle.rope_table(ci.positions) if table is None else table
    return ci, oracle.compress_pack(ci.latent, m, pw, cs, ci.w_idx, intermediates=True)


def test_equal_weights_give_the_fp32_mean():
    n = 64
    w = np.full((2, 512), 0.731, np.float32)
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, pool_w=w)
    x = synth.bf16_bits_to_f32(ci.latent).reshape(n, 2, 512)
    ref = np.mean(x, axis=1, dtype=np.float32)
    assert np.array_equal(pooled.view(np.uint32), ref.view(np.uint32))


def test_m1_is_identity():
    n = 32
    ci, (kv, ix, pooled, rot, k) = _compress(n, 1)
    assert np.array_equal(pooled, synth.bf16_bits_to_f32(ci.latent))


def test_pooling_is_convex_and_matches_quotient_formula():
    n = 128
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, seed=3)
    x = synth.bf16_bits_to_f32(ci.latent).reshape(n, 2, 512).astype(np.float64)
    lo, hi = x.min(axis=1), x.max(axis=1)
    # convex in exact arithmetic; the rounded weighted sum may step one ulp outside
    ulp = np.spacing(np.maximum(np.abs(lo), np.abs(hi)).astype(np.float32)).astype(np.float64)
    assert np.all(pooled >= lo - ulp) and np.all(pooled <= hi + ulp)
    w = ci.pool_w.astype(np.float64)
    quot = (w[0] * x[:, 0] + w[1] * x[:, 1]) / (w[0] + w[1])
    assert np.max(np.abs(pooled - quot)) <= 4 * np.finfo(np.float32).eps * np.max(np.abs(x))


def test_per_token_weights_repeating_the_static_rows_give_the_static_result():
    # per-token gates ([DF] §4.2: the pooling weights may be projected from the input) use the
    # static formula with each token's own row: rows that repeat the static weights reproduce
    # the static entries bit for bit
    n = 96
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, seed=31)
    w_tok = np.tile(ci.pool_w, (n, 1))
    kv2, ix2, pooled2, _, _ = oracle.compress_pack(ci.latent, 2, w_tok, oracle.rope_table(ci.positions), ci.w_idx,
                                                   intermediates=True)
    assert np.array_equal(kv2, kv) and np.array_equal(ix2, ix) and np.array_equal(pooled2, pooled)


def test_per_token_equal_weights_give_the_fp32_mean():
    # a different positive constant per token pair: each entry is still exactly the fp32 mean
    n = 64
    ci = synth.compress_inputs(32, n, 2)
    c = np.exp2(RNG.integers(-20, 20, n)).astype(np.float32) * np.float32(0.37)
    w_tok = np.repeat(np.repeat(c, 2)[:, None], 512, axis=1).astype(np.float32)
    _, _, pooled, _, _ = oracle.compress_pack(ci.latent, 2, w_tok, oracle.rope_table(ci.positions), ci.w_idx,
                                              intermediates=True)
    x = synth.bf16_bits_to_f32(ci.latent).reshape(n, 2, 512)
    assert np.array_equal(pooled.view(np.uint32), np.mean(x, axis=1, dtype=np.float32).view(np.uint32))


def test_per_token_weights_belong_to_their_own_entry():
    # entry j of a per-token call equals a one-entry static call with rows 2j, 2j+1 as weights;
    # swapping an entry's two latents together with their weight rows changes nothing
    n = 24
    ci = synth.compress_inputs(33, n, 2)
    w_tok = synth.softplus_weights(np.random.default_rng(7), 2 * n)
    cs = oracle.rope_table(ci.positions)
    kv, ix = oracle.compress_pack(ci.latent, 2, w_tok, cs, ci.w_idx)
    for j in (0, 5, n - 1):
        kv1, ix1 = oracle.compress_pack(ci.latent[2 * j:2 * j + 2], 2, w_tok[2 * j:2 * j + 2], cs[j:j + 1], ci.w_idx)
        assert np.array_equal(kv1[0], kv[j]) and np.array_equal(ix1[0], ix[j])
    sw = np.arange(2 * n).reshape(n, 2)[:, ::-1].reshape(-1)
    kv_s, ix_s = oracle.compress_pack(ci.latent[sw], 2, w_tok[sw], cs, ci.w_idx)
    assert np.array_equal(kv_s, kv) and np.array_equal(ix_s, ix)
    # a zero weight on one token selects the other token exactly (the convex-combination ends)
    w_sel = w_tok.copy()
    w_sel[1::2] = 0.0
    _, _, pooled, _, _ = oracle.compress_pack(ci.latent, 2, w_sel, cs, ci.w_idx, intermediates=True)
    assert np.array_equal(pooled, synth.bf16_bits_to_f32(ci.latent)[0::2])


def test_rope_position_zero_identity_and_norm():
    n = 16
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, table=rope_id_table(n))
    assert np.array_equal(pooled, rot)
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, seed=9)
    assert np.array_equal(pooled[:, :448], rot[:, :448])  # NoPE channels untouched
    nb = np.linalg.norm(pooled[:, 448:].astype(np.float64).reshape(n, 32, 2), axis=2)
    na = np.linalg.norm(rot[:, 448:].astype(np.float64).reshape(n, 32, 2), axis=2)
    assert np.max(np.abs(na - nb) / np.maximum(nb, 1e-30)) < 4e-7


def test_rope_rotation_is_complex_multiplication():
    n = 40
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, seed=11)
    ang = ci.positions[:, None].astype(np.float64) * 160000.0 ** (-np.arange(32) * 2 / 64.0)
    z = pooled[:, 448:].astype(np.float64).reshape(n, 32, 2)
    zc = (z[..., 0] + 1j * z[..., 1]) * np.exp(1j * ang)
    got = rot[:, 448:].astype(np.float64).reshape(n, 32, 2)
    err = np.abs(got[..., 0] - zc.real) + np.abs(got[..., 1] - zc.imag)
    assert np.max(err) < 2e-6


def test_rope_table_vs_numpy():
    pos = np.array([0, 1, 2, 1000, 65536, 1048574, 2 ** 21], np.int64)
    t = oracle.rope_table(pos)
    ang = pos[:, None].astype(np.float64) * 160000.0 ** (-np.arange(32) * 2 / 64.0)
    ref = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    assert np.max(np.abs(t - ref)) <= 2 * np.finfo(np.float32).eps
    assert np.all(t[0, :32] == 1.0) and np.all(t[0, 32:] == 0.0)


def test_main_kv_pack_layout_and_bounds():
    n = 200
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, seed=5)
    assert kv.shape == (n, 288) and ix.shape == (n, 68)
    # scale byte = torch's nearest-even E4M3 of fp32(amax / 6)
    amax = np.abs(rot.reshape(n, 32, 16)).max(axis=2)
    sraw = (amax / np.float32(6.0)).astype(np.float32)
    ref = torch.from_numpy(sraw).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kv[:, 256:], ref)
    # round trip: every element within one scale step (largest half-gap: 4 -> 6)
    deq = oracle.dequant_kv(kv)
    S = np.repeat(np.array([[oracle.e4m3_value(b) for b in row] for row in kv[:, 256:]]), 16, axis=1)
    assert np.all(np.abs(deq - rot) <= S + 1e-30)
    # the element with the group maximum magnitude keeps its sign
    idx = np.argmax(np.abs(rot.reshape(n, 32, 16)), axis=2)
    sel = np.take_along_axis(rot.reshape(n, 32, 16), idx[..., None], 2)[..., 0]
    dsel = np.take_along_axis(deq.reshape(n, 32, 16), idx[..., None], 2)[..., 0]
    assert np.all(np.sign(sel) == np.sign(dsel))


def test_main_kv_nibble_order_and_2688_saturation():
    # a hand-built pooled vector fed through m = 1 with a position-0 table
    x = np.zeros((1, 512), np.float32)
    x[0, 0], x[0, 1] = 6.0, -0.5  # group 0: amax 6 -> scale 1.0 -> codes 7 and 8|1
    x[0, 16] = 2688.0  # group 1: the largest representable magnitude
    x[0, 32] = 5000.0  # group 2: saturates to 2688
    x[0, 33] = -1.0
    lat = synth.f32_to_bf16_bits(x)
    w = np.zeros((128, 512), np.uint16)
    kv, ix = oracle.compress_pack(lat, 1, None, rope_id_table(1), w)
    assert kv[0, 0] == 0x97
    assert kv[0, 256] == oracle.e4m3_encode(1.0)
    assert kv[0, 257] == 0x7E and (kv[0, 8] & 15) == 7
    deq = oracle.dequant_kv(kv)[0]
    assert deq[16] == 2688.0 and deq[32] == 2688.0
    assert deq[0] == 6.0 and deq[1] == -0.5


def test_indexer_projection_and_mxfp4():
    n = 50
    ci, (kv, ix, pooled, rot, k) = _compress(n, 2, seed=8)
    W = synth.bf16_bits_to_f32(ci.w_idx).astype(np.float64)
    ref = rot.astype(np.float64) @ W.T
    assert np.max(np.abs(k - ref)) < 1e-4 * np.max(np.abs(ref))
    codes = ix[:, 64:].astype(np.int64)
    amax = np.abs(k.reshape(n, 4, 32)).max(axis=2)
    X = np.exp2(codes - 127.0)
    assert np.all((4 * X <= amax) & (amax < 8 * X))
    deq = oracle.dequant_idx(ix)
    Xr = np.repeat(X, 32, axis=1)
    # MX clamps |k| in (6X, 8X) to 6X (error < 2X); below 6X the half-gap bound X holds
    sat = np.abs(k) > 6 * Xr
    assert np.all(np.abs(deq - k)[~sat] <= Xr[~sat])
    assert np.all(np.abs(deq - k)[sat] < 2 * Xr[sat]) and np.all(np.abs(deq[sat]) == 6 * Xr[sat])


def test_indexer_projection_selects_channels_exactly():
    # rows of W with a single 1.0 pick one post-RoPE channel: k equals that channel exactly
    n = 8
    ci = synth.compress_inputs(21, n, 2)
    w = np.zeros((128, 512), np.float32)
    for o in range(128):
        w[o, (o * 3) % 448] = 1.0
    kv, ix, pooled, rot, k = oracle.compress_pack(ci.latent, 2, ci.pool_w, oracle.rope_table(ci.positions),
                                                  synth.f32_to_bf16_bits(w), intermediates=True)
    assert np.array_equal(k, rot[:, [(o * 3) % 448 for o in range(128)]])


# ------------------------------------------------------------------ stage 2: indexer
def _ones_entry(code=0x22, scale=127):
    e = np.zeros(68, np.uint8)
    e[:64] = code  # every nibble = 2 -> value 1.0
    e[64:] = scale  # X = 2^0
    return e


def test_index_score_single_head_all_ones_key():
    q = synth.f32_to_bf16_bits(RNG.standard_normal((1, 32, 128)).astype(np.float32))
    w = np.zeros((1, 32), np.float32)
    w[0, 5] = 1.0
    cache = _ones_entry()[None]
    s = oracle.index_score(q, w, cache, [0], [1], 1)
    qs = synth.bf16_bits_to_f32(q)[0, 5].astype(np.float64).sum()
    assert s[0, 0] == np.float32(max(qs, 0.0))
    cache2 = _ones_entry(code=0xAA)[None]  # every nibble = -1.0
    s2 = oracle.index_score(q, w, cache2, [0], [1], 1)
    assert s2[0, 0] == np.float32(max(-qs, 0.0))


def test_index_score_relu_homogeneity_and_layout():
    n, width = 300, 320
    kv, ix = synth.random_caches(2, n)
    d = synth.query_inputs(3, 2)
    s = oracle.index_score(d.q_idx, d.head_w, ix, [0, 0], [n, 257], width)
    assert np.all(np.isneginf(s[0, n:])) and np.all(np.isneginf(s[1, 257:]))
    # scaling q by 2 (exact in bf16) doubles every score exactly
    q2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(d.q_idx) * 2)
    s2 = oracle.index_score(q2, d.head_w, ix, [0, 0], [n, 257], width)
    assert np.array_equal(s2[:, :257], 2 * s[:, :257])
    # negative q flips every dot product; with non-negative weights ReLU gives 0 then
    qn = synth.f32_to_bf16_bits(-np.abs(synth.bf16_bits_to_f32(d.q_idx)))
    pos_only = np.ones_like(d.head_w)
    pos_cache = ix.copy()
    pos_cache[:, :64] &= 0x77  # clear every sign bit: all key values >= 0
    s3 = oracle.index_score(qn, pos_only, pos_cache, [0, 0], [n, n], width)
    assert np.all(s3[:, :n] == 0)
    # numpy library matmul on the exactly dequantised keys
    kd = oracle.dequant_idx(ix)
    qf = synth.bf16_bits_to_f32(d.q_idx).astype(np.float64)
    ref = np.einsum("thd,jd->thj", qf, kd)
    ref = np.einsum("th,thj->tj", d.head_w.astype(np.float64), np.maximum(ref, 0))
    assert np.allclose(s[0, :n], ref[0], rtol=1e-6, atol=1e-6)


def test_index_score_pool_layout_matches_full():
    n = 200
    kv, ix = synth.random_caches(4, 2 * n)
    d = synth.query_inputs(5, 2)
    base = [0, n]
    full = oracle.index_score(d.q_idx, d.head_w, ix, base, [n, n - 3], n)
    pool = np.array([[0, 3, 24, -1], [24, 2, -1, 5]], np.int32)  # last block of row 1 is partial
    sp = oracle.index_score(d.q_idx, d.head_w, ix, base, [n, n - 3], 32, pool_blocks=pool)
    for t in range(2):
        for slot in range(4):
            for o in range(8):
                b = pool[t, slot]
                j = b * 8 + o
                v = sp[t, slot * 8 + o]
                if b < 0 or j >= (n if t == 0 else n - 3):
                    assert np.isneginf(v)
                else:
                    assert v == full[t, j]


# ------------------------------------------------------------------ stage 3: selection
def np_topk(row, n, K):
    """numpy sort: K largest of row[:n] (NaN as -inf), ties to the lower index, ascending."""
    r = np.where(np.isnan(row[:n]), -np.inf, row[:n]).astype(np.float64)
    order = np.lexsort((np.arange(n), -r))
    return np.sort(order[:K])


def np_pool(row, n, M, block=8):
    """the page's pad / unflatten / amax chain, newest block +inf, numpy top-M blocks."""
    nb = -(-n // block)
    r = np.where(np.isnan(row[:n]), -np.inf, row[:n]).astype(np.float64)
    padded = np.concatenate([r, np.full(nb * block - n, -np.inf)])
    g = padded.reshape(nb, block).max(axis=1)
    g[nb - 1] = np.inf
    order = np.lexsort((np.arange(nb), -g))
    return np.sort(order[:M])


@pytest.mark.parametrize("levels,tie_frac,nan_frac", [(0, 0.0, 0.0), (0, 0.2, 0.0), (6, 0.0, 0.0), (0, 0.1, 0.02)])
def test_pool_covering_all_blocks_equals_bruteforce(levels, tie_frac, nan_frac):
    width = 2048  # 256 blocks <= M
    s = synth.random_scores(17, 3, width, tie_frac=tie_frac, levels=levels, nan_frac=nan_frac)
    nvis = np.array([2048, 2043, 1001], np.int32)
    pool, topk = oracle.block_topk(s, nvis, K=512, M=2048)
    for t in range(3):
        nb = -(-nvis[t] // 8)
        assert np.array_equal(pool[t, :nb], np.arange(nb)) and np.all(pool[t, nb:] == -1)
        assert np.array_equal(topk[t], np_topk(s[t], nvis[t], 512))


@pytest.mark.parametrize("levels,tie_frac", [(0, 0.0), (0, 0.3), (5, 0.0)])
def test_full_layer_hierarchical_equals_global_topk(levels, tie_frac):
    width = 40000  # 5000 blocks > M = 2048
    s = synth.random_scores(19, 2, width, tie_frac=tie_frac, levels=levels)
    nvis = np.array([40000, 39995], np.int32)
    pool, topk = oracle.block_topk(s, nvis, K=512, M=2048)
    for t in range(2):
        assert np.array_equal(pool[t], np_pool(s[t], nvis[t], 2048))
        assert np.array_equal(topk[t], np_topk(s[t], nvis[t], 512))
        nb = -(-nvis[t] // 8)
        assert nb - 1 in pool[t]  # the newest block always takes a slot
        assert np.all(np.diff(pool[t]) > 0)
    assert np.array_equal(topk, oracle.topk_bruteforce(s, nvis, 512))


def test_candidate_mode_is_topk_inside_pool():
    width, M = 12000, 64
    s = synth.random_scores(23, 2, width, tie_frac=0.1)
    nvis = np.array([12000, 11997], np.int32)
    pool, _ = oracle.block_topk(s, nvis, K=512, M=M)
    # lay the pool's scores out as the indexer does in candidate mode
    cand = np.full((2, 8 * M), -np.inf, np.float32)
    for t in range(2):
        for slot, b in enumerate(pool[t]):
            for o in range(8):
                j = b * 8 + o
                if b >= 0 and j < nvis[t]:
                    cand[t, slot * 8 + o] = s[t, j]
    _, topk = oracle.block_topk(cand, nvis, K=100, pool_blocks=pool)
    for t in range(2):
        ids = np.concatenate([np.arange(b * 8, b * 8 + 8) for b in pool[t] if b >= 0])
        ids = ids[ids < nvis[t]]
        order = np.lexsort((ids, -s[t, ids].astype(np.float64)))
        assert np.array_equal(topk[t], np.sort(ids[order[:100]]))


def test_pool_size_bound_and_short_rows():
    s = synth.random_scores(29, 3, 1000)
    nvis = np.array([0, 5, 300], np.int32)
    pool, topk = oracle.block_topk(s, nvis, K=512, M=16)
    assert np.all(pool[0] == -1) and np.all(topk[0] == -1)
    assert np.array_equal(topk[1, :5], np.arange(5)) and np.all(topk[1, 5:] == -1)
    assert np.array_equal(pool[1, :1], [0]) and np.all(pool[1, 1:] == -1)
    assert np.sum(pool[2] >= 0) == 16 and 37 in pool[2]
    # 15 full blocks plus the newest block, of which only positions 296..299 are visible
    assert np.sum(topk[2] >= 0) == 15 * 8 + 4
    # a negative visible count sees nothing, as a zero count does
    pool_n, topk_n = oracle.block_topk(s, np.array([-9, -1, 300], np.int32), K=512, M=16)
    assert np.all(pool_n[:2] == -1) and np.all(topk_n[:2] == -1)
    assert np.array_equal(pool_n[2], pool[2]) and np.array_equal(topk_n[2], topk[2])
    assert np.all(oracle.topk_bruteforce(s, np.array([-3, 0, 0], np.int32), 512) == -1)


# ------------------------------------------------------------------ stage 4: attention
def _attn_case(seed, nsel, nswa, n_entries=64):
    kv, ix = synth.random_caches(seed, n_entries)
    d = synth.query_inputs(seed + 1, 1, swa_rows=128)
    rng = np.random.default_rng(seed)
    topk = np.full((1, 512), -1, np.int32)
    topk[0, :nsel] = np.sort(rng.choice(n_entries, nsel, replace=False))
    return kv, d, topk, np.array([nswa], np.int32)


def test_attention_zero_query_is_mean_of_keys():
    kv, d, topk, sl = _attn_case(31, 40, 100)
    q0 = np.zeros_like(d.q)
    out, lse = oracle.sparse_attn(q0, kv, [0], topk, d.swa, d.swa_start, sl)
    keys = np.concatenate([oracle.dequant_kv(kv[topk[0, :40]]),
                           synth.bf16_bits_to_f32(d.swa[:100]).astype(np.float64)])
    ref = keys.mean(axis=0)
    assert np.max(np.abs(out[0] - ref[None])) < 1e-6 * np.max(np.abs(ref))
    assert np.allclose(lse[0], np.log(140.0), rtol=1e-6)


def test_attention_single_key_and_empty():
    kv, d, topk, sl = _attn_case(33, 1, 0)
    out, lse = oracle.sparse_attn(d.q, kv, [0], topk, d.swa, d.swa_start, sl)
    key = oracle.dequant_kv(kv[topk[0, 0]])[0]
    assert np.array_equal(out[0], np.broadcast_to(key.astype(np.float32), (64, 512)))
    topk[:] = -1
    out, lse = oracle.sparse_attn(d.q, kv, [0], topk, d.swa, d.swa_start, sl)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_attention_convex_hull_and_order_invariance():
    kv, d, topk, sl = _attn_case(35, 300, 128, n_entries=400)
    out, lse = oracle.sparse_attn(d.q, kv, [0], topk, d.swa, d.swa_start, sl)
    keys = np.concatenate([oracle.dequant_kv(kv[topk[0, :300]]),
                           synth.bf16_bits_to_f32(d.swa[:128]).astype(np.float64)])
    lo, hi = keys.min(axis=0), keys.max(axis=0)
    assert np.all(out[0] >= lo - 1e-6) and np.all(out[0] <= hi + 1e-6)
    perm = topk.copy()
    perm[0, :300] = np.random.default_rng(0).permutation(topk[0, :300])
    out2, _ = oracle.sparse_attn(d.q, kv, [0], perm, d.swa, d.swa_start, sl)
    assert np.allclose(out, out2, rtol=1e-6, atol=1e-7)


def test_attention_common_logit_shift_is_invisible():
    # every key has the same value in channel 7, so adding delta * e_7 to q shifts all
    # logits by the same amount; the softmax, hence the output, must not move
    kv, d, topk, sl = _attn_case(37, 50, 0)
    for e in topk[0, :50]:
        kv[e, 3] = (kv[e, 3] & 0x0F) | 0x40  # channel 7 code = 4 (2.0) ...
        kv[e, 256] = 0x38  # ... with group-0 scale 1.0
    q = synth.bf16_bits_to_f32(d.q).copy()
    q2 = q.copy()
    q2[0, :, 7] += 3.0
    o1, l1 = oracle.sparse_attn(synth.f32_to_bf16_bits(q), kv, [0], topk, d.swa, d.swa_start, sl)
    o2, l2 = oracle.sparse_attn(synth.f32_to_bf16_bits(q2), kv, [0], topk, d.swa, d.swa_start, sl)
    assert np.allclose(o1, o2, rtol=1e-5, atol=1e-6)
    shift = 3.0 * 2.0 / np.sqrt(512.0)
    q2b = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(q2))
    qb = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(q))
    exact_shift = (q2b[0, :, 7] - qb[0, :, 7]).astype(np.float64) * 2.0 / np.sqrt(512.0)
    assert np.allclose(l2[0] - l1[0], exact_shift, atol=1e-4)
    assert abs(np.mean(exact_shift) - shift) < 0.05


def test_attention_scale_is_on_the_logits():
    kv, d, topk, sl = _attn_case(39, 64, 64)
    q2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(d.q) * 2)  # exact
    o1, l1 = oracle.sparse_attn(d.q, kv, [0], topk, d.swa, d.swa_start, sl, scale=0.05)
    o2, l2 = oracle.sparse_attn(q2, kv, [0], topk, d.swa, d.swa_start, sl, scale=0.025)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_attention_two_keys_closed_form():
    # two keys differing only in channel 0: weights are a logistic of the logit gap
    kv = np.zeros((2, 288), np.uint8)
    kv[:, 256:] = 0x38  # all scales 1.0
    kv[0, 0] = 0x07  # channel 0 = 6.0
    kv[1, 0] = 0x02  # channel 0 = 1.0
    q = np.zeros((1, 64, 512), np.float32)
    q[0, :, 0] = np.linspace(-2, 2, 64, dtype=np.float32)
    qb = synth.f32_to_bf16_bits(q)
    topk = np.full((1, 512), -1, np.int32)
    topk[0, :2] = [0, 1]
    swa = np.zeros((1, 512), np.uint16)
    out, _ = oracle.sparse_attn(qb, kv, [0], topk, swa, [0], [0])
    qv = synth.bf16_bits_to_f32(qb)[0, :, 0].astype(np.float64)
    gap = qv * (6.0 - 1.0) / np.sqrt(512.0)
    p0 = 1.0 / (1.0 + np.exp(-gap))
    assert np.allclose(out[0, :, 0], 6.0 * p0 + 1.0 * (1 - p0), rtol=1e-6)
    assert np.all(out[0, :, 1:] == 0)
