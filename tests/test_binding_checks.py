"""CPU checks of the Python binding's argument validation: every wrapper rejects a tensor
of the wrong shape, dtype or layout with ValueError before the library is called.

The device predicate and the library handle are replaced for the test (host tensors stand
in for device tensors; the stand-in library records calls and launches nothing), so this
runs without a GPU.  A call with every shape right must reach the library exactly once."""
import types

import pytest
import torch

from fp4_kv_cache_csa2_amd import csa2

BF, F32, U8, I32, I64 = torch.bfloat16, torch.float32, torch.uint8, torch.int32, torch.int64


class FakeLib:
    def __init__(self, real):
        self.calls = []
        self.real = real

    def __getattr__(self, name):
        if name.endswith("_workspace"):
            return getattr(self.real, name)  # host-only size queries
        if name == "csa2_status_string":
            return self.real.csa2_status_string

        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture()
def fake(monkeypatch):
    lib = FakeLib(csa2._L)
    monkeypatch.setattr(csa2, "_L", lib)
    monkeypatch.setattr(csa2, "_is_device", lambda t: True)
    monkeypatch.setattr(csa2, "_stream", lambda s: None)
    return lib


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def expect_ok(lib, fn, **kw):
    n = len(lib.calls)
    fn(**kw)
    assert len(lib.calls) == n + 1, "a valid call must reach the library once"


def expect_bad(lib, fn, **kw):
    n = len(lib.calls)
    with pytest.raises(ValueError):
        fn(**kw)
    assert len(lib.calls) == n, "a rejected call must not reach the library"


def test_compress_checks(fake):
    n, m = 8, 2
    good = dict(latent=z((n * m, 512), BF), m=m, pool_w=z((m, 512), F32), rope_cs=z((n, 64), F32),
                w_idx=z((128, 512), BF), kv_out=z((n, 288), U8), idx_out=z((1, 2176), U8))
    expect_ok(fake, csa2.compress_pack, **good)
    expect_ok(fake, csa2.compress_pack, **{**good, "pool_w": z((n * m, 512), F32)})  # per-token weights
    for k, v in (("latent", z((n * m + 1, 512), BF)), ("latent", z((n * m, 256), BF)), ("pool_w", z((3, 512), F32)),
                 ("pool_w", None), ("rope_cs", z((n - 1, 64), F32)), ("w_idx", z((128, 511), BF)),
                 ("kv_out", z((n - 1, 288), U8)), ("idx_out", z((n, 68), U8)), ("idx_out", z((0, 2176), U8)),
                 ("pool_w", z((m, 512), torch.float64)),
                 ("latent", z((512, n * m), BF).t())):
        expect_bad(fake, csa2.compress_pack, **{**good, k: v})
    app = dict(latent=good["latent"], m=m, pool_w=good["pool_w"], rope_cs=good["rope_cs"], w_idx=good["w_idx"],
               dst_rows=z((n,), I64), kv_cache=z((100, 288), U8), idx_cache=z((4, 2176), U8))
    expect_ok(fake, csa2.compress_append, **app)
    for k, v in (("dst_rows", z((n + 1,), I64)), ("dst_rows", None), ("kv_cache", z((100, 68), U8)),
                 ("idx_cache", z((4 * 2176,), U8)), ("idx_cache", z((100, 68), U8))):
        expect_bad(fake, csa2.compress_append, **{**app, k: v})


def test_index_score_checks(fake):
    n_q, width, M = 3, 1000, 16
    good = dict(q_idx=z((n_q, 32, 128), BF), head_w=z((n_q, 32), F32), idx_cache=z((157, 2176), U8),
                q_base=z((n_q,), I64), q_nvis=z((n_q,), I32), width=width, scores=z((n_q, width), F32),
                block_max=z((n_q, (width + 7) // 8), F32))
    expect_ok(fake, csa2.index_score, **good)
    for k, v in (("q_idx", z((n_q, 32, 64), BF)), ("head_w", z((n_q + 1, 32), F32)), ("q_base", z((n_q - 1,), I64)),
                 ("q_nvis", z((n_q,), I64)), ("scores", z((n_q, width - 1), F32)),
                 ("block_max", z((n_q, width // 8 - 1), F32)), ("idx_cache", z((5000, 68), U8))):
        expect_bad(fake, csa2.index_score, **{**good, k: v})
    cand = {**good, "width": 8 * M, "pool_blocks": z((n_q, M), I32), "scores": z((n_q, 8 * M), F32),
            "block_max": None, "want_block_max": False}
    expect_ok(fake, csa2.index_score, **cand)
    expect_bad(fake, csa2.index_score, **{**cand, "width": 8 * M + 8, "scores": z((n_q, 8 * M + 8), F32)})
    expect_bad(fake, csa2.index_score, **{**cand, "pool_blocks": z((n_q + 1, M), I32)})
    fq = {**good, "q_fp4": z((n_q, 32, 68), U8)}
    del fq["q_idx"]
    expect_ok(fake, csa2.index_score_fp4q, **fq)
    expect_bad(fake, csa2.index_score_fp4q, **{**fq, "q_fp4": z((n_q, 32, 64), U8)})
    expect_ok(fake, csa2.quantize_q_mxfp4, q_idx=z((n_q, 32, 128), BF), out=z((n_q, 32, 68), U8))
    expect_bad(fake, csa2.quantize_q_mxfp4, q_idx=z((n_q, 32, 128), BF), out=z((n_q, 31, 68), U8))


def test_append_index_checks(fake):
    n_q, m, width = 4, 2, 4096
    good = dict(latent=z((n_q * m, 512), BF), m=m, pool_w=z((m, 512), F32), rope_cs=z((n_q, 64), F32),
                w_idx=z((128, 512), BF), kv_cache=z((width * n_q, 288), U8), idx_cache=z((width * n_q // 32, 2176), U8),
                q_idx=z((n_q, 32, 128), BF), head_w=z((n_q, 32), F32), q_base=z((n_q,), I64),
                q_nvis=z((n_q,), I32), width=width)
    expect_ok(fake, csa2.append_index_score, **good)
    expect_ok(fake, csa2.append_index_score, **{**good, "pool_w": z((n_q * m, 512), F32)})
    expect_ok(fake, csa2.append_index_score, **{**good, "q_idx": z((n_q, 32, 68), U8)})
    for k, v in (("latent", z(((n_q + 1) * m, 512), BF)), ("pool_w", z((n_q * m + 2, 512), F32)),
                 ("rope_cs", z((n_q - 1, 64), F32)), ("head_w", z((n_q, 31), F32)), ("q_nvis", z((n_q + 1,), I32)),
                 ("scores", z((n_q, width + 1), F32)), ("block_max", z((n_q, 1), F32)),
                 ("q_idx", z((n_q, 32, 60), U8))):
        expect_bad(fake, csa2.append_index_score, **{**good, k: v})
    # the variant that counts the selection's first pass: bf16 query, block maxima, a large
    # enough selection workspace
    sel = {**good, "sel_workspace": z((n_q * 4096 * 4,), U8)}
    expect_ok(fake, csa2.append_index_score, **sel)
    assert fake.calls[-1] == "csa2_append_index_score_sel"
    for k, v in (("q_idx", z((n_q, 32, 68), U8)), ("pack_q", True), ("want_block_max", False),
                 ("sel_workspace", z((n_q * 4096 * 4 - 4,), U8))):
        expect_bad(fake, csa2.append_index_score, **{**sel, k: v})
    mean = {**good, "mean_cache": z((width // 32, 2176), U8), "mean_base": z((n_q,), I64)}
    expect_ok(fake, csa2.append_mean_index_score, **mean)
    expect_bad(fake, csa2.append_mean_index_score, **{**mean, "mean_base": z((n_q + 1,), I64)})
    expect_bad(fake, csa2.append_mean_index_score, **{**mean, "mean_cache": z((width, 68), U8)})


def test_block_topk_checks(fake):
    n_q, width, M, K = 2, 4000, 64, 32
    good = dict(scores=z((n_q, width), F32), q_nvis=z((n_q,), I32), K=K, M=M, block_max=z((n_q, 500), F32),
                pool_out=z((n_q, M), I32), topk_out=z((n_q, K), I32))
    expect_ok(fake, csa2.block_topk, **good)
    for k, v in (("q_nvis", z((n_q + 1,), I32)), ("block_max", z((n_q, 499), F32)), ("pool_out", z((n_q, M - 1), I32)),
                 ("topk_out", z((n_q, K + 1), I32)), ("scores", z((n_q, width), torch.float16))):
        expect_bad(fake, csa2.block_topk, **{**good, k: v})
    cand = dict(scores=z((n_q, 8 * M), F32), q_nvis=z((n_q,), I32), K=K, pool_blocks=z((n_q, M), I32),
                topk_out=z((n_q, K), I32))
    expect_ok(fake, csa2.block_topk, **cand)
    expect_bad(fake, csa2.block_topk, **{**cand, "scores": z((n_q, 8 * M + 8), F32)})
    expect_bad(fake, csa2.block_topk, **{**cand, "pool_blocks": z((n_q + 1, M), I32)})
    # the selection after the first-pass handoff: Full mode, block maxima and a full workspace
    ws = z((csa2.block_topk_workspace(n_q, width, M, K),), U8)
    pre = {**good, "workspace": ws, "hist_ready": True}
    expect_ok(fake, csa2.block_topk, **pre)
    assert fake.calls[-1] == "csa2_block_topk_prebuilt"
    for k, v in (("block_max", None), ("workspace", None), ("workspace", z((ws.numel() - 4,), U8))):
        expect_bad(fake, csa2.block_topk, **{**pre, k: v})
    expect_bad(fake, csa2.block_topk, **{**cand, "workspace": ws, "hist_ready": True})
    pool_only = dict(scores=None, q_nvis=z((n_q,), I32), K=K, M=M, block_max=z((n_q, 500), F32),
                     pool_out=z((n_q, M), I32), want_topk=False)
    expect_ok(fake, csa2.block_topk, **pool_only)
    expect_bad(fake, csa2.block_topk, **{**pool_only, "pool_out": z((n_q + 1, M), I32)})


def test_block_mean_pack_checks(fake):
    n_seq = 3
    good = dict(idx_cache=z((25, 2176), U8), seq_base=z((n_seq,), I64), seq_n=z((n_seq,), I32), n_blocks=4,
                mean_cache=z((4, 2176), U8), mean_base=z((n_seq,), I64))
    expect_ok(fake, csa2.block_mean_pack, **good)
    for k, v in (("seq_n", z((n_seq + 1,), I32)), ("mean_base", z((n_seq,), I32)), ("first_block", z((1,), I32)),
                 ("mean_cache", z((100, 68), U8))):
        expect_bad(fake, csa2.block_mean_pack, **{**good, k: v})


def test_sparse_attn_checks(fake):
    n_q, K = 3, 40
    good = dict(q=z((n_q, 64, 512), BF), kv_cache=z((1000, 288), U8), q_base=z((n_q,), I64),
                topk=z((n_q, K), I32), swa=z((400, 512), BF), swa_start=z((n_q,), I64), swa_len=z((n_q,), I32),
                out=z((n_q, 64, 512), F32), lse=z((n_q, 64), F32))
    expect_ok(fake, csa2.sparse_attn, **good)
    for k, v in (("q", z((n_q, 32, 512), BF)), ("topk", z((n_q + 1, K), I32)), ("swa", z((400, 256), BF)),
                 ("swa_start", z((n_q - 1,), I64)), ("swa_len", z((n_q,), I64)), ("out", z((n_q, 64, 511), F32)),
                 ("lse", z((n_q, 65), F32)), ("kv_cache", z((1000, 68), U8)), ("q_base", None)):
        expect_bad(fake, csa2.sparse_attn, **{**good, k: v})
    f8 = {**good, "swa8": z((400, 584), U8), "swa_ring": 128}
    del f8["swa"]
    expect_ok(fake, csa2.sparse_attn_swa_fp8, **f8)
    expect_bad(fake, csa2.sparse_attn_swa_fp8, **{**f8, "swa8": z((400, 512), U8)})
    expect_ok(fake, csa2.swa_pack_fp8, rows=z((5, 512), BF), out=z((5, 584), U8))
    expect_bad(fake, csa2.swa_pack_fp8, rows=z((5, 512), BF), out=z((4, 584), U8))
    expect_bad(fake, csa2.swa_pack_fp8, rows=z((5, 512), BF), out=z((10, 584), U8), dst_rows=z((4,), I64))
