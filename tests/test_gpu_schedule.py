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
from tests.gpu_util import bf16, check_attn, dev, host

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def test_decode_schedule_two_tokens():
    from fp4_kv_cache_csa2_amd import schedule as gsched
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    n_seq, tokens, K, M = 2, 2000, 32, 40
    cap = tokens + 4
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
        assert np.array_equal(host(g.kv[c]), ocs.kv[c]) and np.array_equal(host(g.ix[c]), ocs.ix[c]), c
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
            assert np.array_equal(host(g.kv[c]), ocs.kv[c]) and np.array_equal(host(g.ix[c]), ocs.ix[c]), c
        for l in layers:
            rel = check_attn(host(outs[l]), ref[l][0])
            assert np.allclose(host(lses[l]), ref[l][1], atol=2e-3), f"layer {l} lse"
        log(f"  {len(layers)} layers match; caches {dict(g.n)}")
