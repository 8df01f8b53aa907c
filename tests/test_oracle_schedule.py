"""Pins for the oracle's 40-layer decode schedule (CPU only): the layer plan against the
counts and source layers the pages print (tests/golden/pages_numbers.txt), the resident
bytes per token the plan's caches imply, and the mode semantics checked through
invariants of a small run — which layer's Top-K a Reuse layer reads, when each cache
grows, and that a Reindex layer fed the Full layer's indexer query reselects the Full
layer's set."""
import numpy as np
import pytest

import oracle
from fp4_kv_cache_csa2_amd import synth
from oracle import schedule
from tests.test_oracle_formats import G


def test_plan_matches_the_printed_layer_plan():
    plan = schedule.layer_plan()
    assert len(plan) == G["model_layers"] == 40
    modes = [m for m, _ in plan]
    assert modes[:2] == ["swa", "swa"] and modes.count("swa") == G["swa_only_layers"]
    enc, dec = plan[:20], plan[20:]
    assert len(enc) == G["encoder_layers"] and len(dec) == G["decoder_layers"]
    full = [i for i, (m, _) in enumerate(plan) if m == "full"]
    assert full == [G["kv_source_layer_0based_%d" % k] for k in (1, 2, 3, 4)]
    assert len({c for _, c in plan if c}) == G["kv_source_layers"]
    # Encoder blocks of 6 (Full + 5 Reuse) each on their own cache; Decoder blocks of 4
    for b in range(3):
        blk = plan[2 + 6 * b: 8 + 6 * b]
        assert len(blk) == G["encoder_block_layers"]
        assert blk[0] == ("full", "enc%d" % b) and all(x == ("reuse", "enc%d" % b) for x in blk[1:])
    for b in range(5):
        blk = dec[4 * b: 4 * b + 4]
        assert len(blk) == G["decoder_block_layers"]
        assert blk[0] == (("full" if b == 0 else "reindex"), "dec") and all(x == ("reuse", "dec") for x in blk[1:])
    assert modes.count("reuse") == 30 and modes.count("reindex") == 4


def test_plan_caches_give_890_bytes_per_token():
    caches = {c for _, c in schedule.layer_plan() if c}
    per_token = sum((oracle.entry_bytes(512, 16) + oracle.entry_bytes(128, 32)) / schedule.CACHE_RATIO[c]
                    for c in caches)
    assert per_token == G["global_kv_bytes_per_token"]


def _setup(seed, n_seq, tokens, cap):
    rng = np.random.default_rng(seed)
    cs = schedule.SeqCaches(n_seq, cap)
    params, lat = {}, {}
    for i, c in enumerate(schedule.CACHE_RATIO):
        m = schedule.CACHE_RATIO[c]
        ci = synth.compress_inputs(seed + 10 * i, n_seq * (tokens // m), m)
        params[c] = (ci.pool_w, ci.w_idx)
        lat[c] = ci.latent.reshape(n_seq, tokens, 512)
        n = tokens // m
        pos = np.tile(np.arange(n, dtype=np.int64) * m, n_seq)
        kv, ix = oracle.compress_pack(ci.latent, m, ci.pool_w, oracle.rope_table(pos), ci.w_idx)
        for s in range(n_seq):
            cs.kv[c][s * cap: s * cap + n] = kv[s * n:(s + 1) * n]
            cs.ix[c][s * cap: s * cap + n] = ix[s * n:(s + 1) * n]
        cs.n[c] = n
    inputs = {}
    for layer, (mode, c) in enumerate(schedule.layer_plan()):
        if mode == "swa":
            continue
        d = synth.query_inputs(seed + 100 + layer, n_seq, swa_len=np.full(n_seq, 128, np.int32))
        inputs[layer] = {"q": d.q, "swa": d.swa, "swa_len": d.swa_len, "q_idx": d.q_idx, "head_w": d.head_w}
    return rng, cs, params, lat, inputs


def _new_latents(rng, n_seq):
    return {c: synth.f32_to_bf16_bits(rng.standard_normal((n_seq, m, 512)).astype(np.float32))
            for c, m in schedule.CACHE_RATIO.items()}


@pytest.mark.parametrize("p", [2001, 2000])
def test_schedule_modes_and_appends(p):
    n_seq, tokens, K, M = 2, 2000, 32, 40  # M - 1 >= K: the Full Top-K lies inside its pool
    rng, cs, params, lat, inputs = _setup(7 + p, n_seq, tokens, cap=tokens + 4)
    n0 = dict(cs.n)
    # the decoder Reindex layers reuse the Full layer's indexer query: they must reselect
    # the Full layer's set (the Full Top-K equals the Top-K inside its own pool)
    for l in (24, 28, 32, 36):
        inputs[l]["q_idx"], inputs[l]["head_w"] = inputs[20]["q_idx"], inputs[20]["head_w"]
    outs = schedule.decode_token(cs, p, _new_latents(rng, n_seq), params, inputs, K=K, M=M)
    assert sorted(outs) == [l for l, (m, _) in enumerate(schedule.layer_plan()) if m != "swa"]
    for c, m in schedule.CACHE_RATIO.items():  # position p completes an entry iff (p + 1) % m == 0
        assert cs.n[c] == n0[c] + (1 if (p + 1) % m == 0 else 0)
    base = np.arange(n_seq, dtype=np.int64) * cs.cap
    swa_start = np.arange(n_seq, dtype=np.int64) * 128
    for src, reusers, c in [(2, range(3, 8), "enc0"), (8, range(9, 14), "enc1"), (14, range(15, 20), "enc2"),
                            (20, range(21, 24), "dec")]:
        nvis = np.full(n_seq, cs.n[c], np.int32)
        s = oracle.index_score(inputs[src]["q_idx"], inputs[src]["head_w"], cs.ix[c], base, nvis, cs.n[c])
        tk = oracle.topk_bruteforce(s, nvis, K=K)
        for l in [src, *reusers]:
            o, lse = oracle.sparse_attn(inputs[l]["q"], cs.kv[c], base, tk, inputs[l]["swa"], swa_start,
                                        inputs[l]["swa_len"])
            assert np.array_equal(outs[l][0], o) and np.array_equal(outs[l][1], lse), f"layer {l}"
    for x in (24, 28, 32, 36):
        for l in range(x, x + 4):
            np.testing.assert_array_equal(outs[l][0], oracle.sparse_attn(
                inputs[l]["q"], cs.kv["dec"], base, tk, inputs[l]["swa"], swa_start, inputs[l]["swa_len"])[0])
