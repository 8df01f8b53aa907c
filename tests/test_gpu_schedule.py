"""GPU parity of the 40-layer decode schedule (fp4_kv_cache_csa2_amd/schedule.py, through
the C ABI) against the oracle's schedule (oracle/schedule.py), token by token: every CSA2
layer's attention output (tolerance of tests/gpu_util.py) and the caches (bit-exact)
after appends at an even and an odd position."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import synth
from oracle import schedule as osched
from tests.gpu_util import bf16, check_attn, dev, dev_ix, host, host_ix

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def test_decode_schedule_two_tokens():
    from fp4_kv_cache_csa2_amd import schedule as gsched
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    n_seq, tokens, K, M = 2, 2000, 32, 40
    cap = 2016  # whole tiles of 32 entries (the branch rounds its capacities to tiles), room for 2 tokens
    rng = np.random.default_rng(5)
    ocs = osched.SeqCaches(n_seq, cap)
    g = gsched.GlobalBranch(n_seq, {c: cap for c in gsched.RATIO}, K=K, M=M)
    params = {}
    log("schedule: filling caches")
    for i, c in enumerate(osched.CACHE_RATIO):
        m = osched.CACHE_RATIO[c]
        ci = synth.compress_inputs(50 + i, n_seq * tokens // m, m)
        params[c] = (ci.pool_w, ci.w_idx)
        lat = ci.latent.reshape(n_seq, tokens, 512)
        n = tokens // m
        pos = np.tile(np.arange(n, dtype=np.int64) * m, n_seq)
        kv, ix = oracle.compress_pack(ci.latent, m, ci.pool_w, oracle.rope_table(pos), ci.w_idx)
        for s in range(n_seq):
            ocs.kv[c][s * cap: s * cap + n] = kv[s * n:(s + 1) * n]
            ocs.ix[c][s * cap: s * cap + n] = ix[s * n:(s + 1) * n]
        ocs.n[c] = n
        g.set_params(c, dev(ci.pool_w), bf16(ci.w_idx))
        g.fill(c, bf16(lat))
    torch.cuda.synchronize()
    for c in osched.CACHE_RATIO:
        assert np.array_equal(host(g.kv[c]), ocs.kv[c]) and np.array_equal(host_ix(g.ix[c]), ocs.ix[c]), c
    layers = [l for l, (mo, _) in enumerate(osched.layer_plan()) if mo != "swa"]
    assert layers == gsched.csa2_layers()
    for p in (tokens, tokens + 1):
        log(f"schedule: token at position {p}")
        inputs, ginputs = {}, {}
        for l in layers:
            d = synth.query_inputs(1000 * p + l, n_seq, swa_len=rng.integers(1, 129, n_seq).astype(np.int32))
            inputs[l] = {"q": d.q, "swa": d.swa, "swa_len": d.swa_len, "q_idx": d.q_idx, "head_w": d.head_w}
            ginputs[l] = {"q": bf16(d.q), "swa": bf16(d.swa), "swa_start": dev(d.swa_start), "swa_len": dev(d.swa_len),
                          "q_idx": bf16(d.q_idx), "head_w": dev(d.head_w)}
        new = {c: synth.f32_to_bf16_bits(rng.standard_normal((n_seq, m, 512)).astype(np.float32))
               for c, m in osched.CACHE_RATIO.items()}
        outs = {l: torch.empty((n_seq, 64, 512), dtype=torch.float32, device="cuda") for l in layers}
        lses = {l: torch.empty((n_seq, 64), dtype=torch.float32, device="cuda") for l in layers}
        g.decode_token(p, {c: bf16(v.reshape(-1, 512)) for c, v in new.items()}, ginputs, outs, lses)
        torch.cuda.synchronize()
        ref = osched.decode_token(ocs, p, new, params, inputs, K=K, M=M)
        assert g.n == ocs.n
        for c in osched.CACHE_RATIO:
            assert np.array_equal(host(g.kv[c]), ocs.kv[c]) and np.array_equal(host_ix(g.ix[c]), ocs.ix[c]), c
        for l in layers:
            rel = check_attn(host(outs[l]), ref[l][0])
            assert np.allclose(host(lses[l]), ref[l][1], atol=2e-3), f"layer {l} lse"
        log(f"  {len(layers)} layers match; caches {dict(g.n)}")


def test_decode_schedule_full_size_k512_m2048():
    """The 40-layer schedule at the model's K = 512 and M = 2048 on caches larger than the
    pool: 20000 entries in each Encoder cache (m = 2) and 40001 in the Decoder cache (m = 1),
    so the Full layers' pools (2048 blocks of 8 = 16384 positions) cover only part of every
    cache.  The history is drawn directly as packed bytes (the same on both sides); the
    token at position 40001 appends to all four caches, the token at 40002 to the Decoder
    cache only.  Every CSA2 layer's output and the caches are compared."""
    from fp4_kv_cache_csa2_amd import schedule as gsched
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    n_seq, K, M = 2, 512, 2048
    n_hist = {"enc0": 20000, "enc1": 20000, "enc2": 20000, "dec": 40001}
    cap = 40032  # whole tiles of 32 entries
    rng = np.random.default_rng(9)
    ocs = osched.SeqCaches(n_seq, cap)
    g = gsched.GlobalBranch(n_seq, {c: cap for c in gsched.RATIO}, K=K, M=M)
    params = {}
    log("schedule K=512 M=2048: drawing caches")
    for i, c in enumerate(osched.CACHE_RATIO):
        kv, ix = synth.random_caches(80 + i, n_seq * cap)
        for s in range(n_seq):  # rows past the history hold zeros, as appended rows start out
            kv[s * cap + n_hist[c]:(s + 1) * cap] = 0
            ix[s * cap + n_hist[c]:(s + 1) * cap] = 0
        ocs.kv[c][:], ocs.ix[c][:] = kv, ix
        ocs.n[c] = n_hist[c]
        g.kv[c].copy_(dev(kv))
        g.ix[c].copy_(dev_ix(ix))
        g.n[c] = n_hist[c]
        ci = synth.compress_inputs(90 + i, 1, osched.CACHE_RATIO[c])
        params[c] = (ci.pool_w, ci.w_idx)
        g.set_params(c, dev(ci.pool_w), bf16(ci.w_idx))
    torch.cuda.synchronize()
    layers = gsched.csa2_layers()
    for p in (2 * 20000 + 1, 2 * 20000 + 2):
        log(f"schedule K=512 M=2048: token at position {p}")
        inputs, ginputs = {}, {}
        for l in layers:
            d = synth.query_inputs(7000 * p + l, n_seq, swa_len=rng.integers(1, 129, n_seq).astype(np.int32))
            inputs[l] = {"q": d.q, "swa": d.swa, "swa_len": d.swa_len, "q_idx": d.q_idx, "head_w": d.head_w}
            ginputs[l] = {"q": bf16(d.q), "swa": bf16(d.swa), "swa_start": dev(d.swa_start), "swa_len": dev(d.swa_len),
                          "q_idx": bf16(d.q_idx), "head_w": dev(d.head_w)}
        new = {c: synth.f32_to_bf16_bits(rng.standard_normal((n_seq, m, 512)).astype(np.float32))
               for c, m in osched.CACHE_RATIO.items()}
        outs = {l: torch.empty((n_seq, 64, 512), dtype=torch.float32, device="cuda") for l in layers}
        lses = {l: torch.empty((n_seq, 64), dtype=torch.float32, device="cuda") for l in layers}
        g.decode_token(p, {c: bf16(v.reshape(-1, 512)) for c, v in new.items()}, ginputs, outs, lses)
        torch.cuda.synchronize()
        ref = osched.decode_token(ocs, p, new, params, inputs, K=K, M=M)
        assert g.n == ocs.n
        for c in osched.CACHE_RATIO:
            assert np.array_equal(host(g.kv[c]), ocs.kv[c]) and np.array_equal(host_ix(g.ix[c]), ocs.ix[c]), c
        for l in layers:
            check_attn(host(outs[l]), ref[l][0])
            assert np.allclose(host(lses[l]), ref[l][1], atol=2e-3), f"layer {l} lse"
        log(f"  {len(layers)} layers match; caches {dict(g.n)}")


def test_decode_schedule_memory_stays_flat():
    """Eager decoding of 300 consecutive positions allocates no device memory per token (the
    branch refills its own token state in place)."""
    from fp4_kv_cache_csa2_amd import schedule as gsched
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    n_seq, tokens, K, M = 2, 64, 16, 17
    cap = tokens + 320
    g = gsched.GlobalBranch(n_seq, {c: cap for c in gsched.RATIO}, K=K, M=M)
    for i, c in enumerate(gsched.RATIO):
        m = gsched.RATIO[c]
        ci = synth.compress_inputs(60 + i, n_seq * tokens // m, m)
        g.set_params(c, dev(ci.pool_w), bf16(ci.w_idx))
        g.fill(c, bf16(ci.latent.reshape(n_seq, tokens, 512)))
    layers = gsched.csa2_layers()
    d = synth.query_inputs(5, n_seq)
    ginputs = {l: {"q": bf16(d.q), "swa": bf16(d.swa), "swa_start": dev(d.swa_start), "swa_len": dev(d.swa_len),
                   "q_idx": bf16(d.q_idx), "head_w": dev(d.head_w)} for l in layers}
    new = {c: bf16(np.zeros((n_seq * m, 512), np.uint16)) for c, m in gsched.RATIO.items()}
    outs = {l: torch.empty((n_seq, 64, 512), dtype=torch.float32, device="cuda") for l in layers}
    used = []
    for p in range(tokens, tokens + 300):
        g.decode_token(p, new, ginputs, outs)
        if p % 50 == 0:
            torch.cuda.synchronize()
            used.append(torch.cuda.memory_allocated())
    log(f"allocated bytes every 50 tokens: {used}")
    assert max(used) == min(used), "device memory grows with the decoded position"
