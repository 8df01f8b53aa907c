"""The decode schedule of the CSA2 global branch over the 40-layer stack, as a plain
composition of the oracle's stages.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[DF] "4. 层维度(下):CSA2 与每 token 890 字节" §4.3 gives the layer plan and the three
modes: Full writes its main KV and indexer K and computes a Top-K; Reindex reads the
latest Main KV / indexer K and recomputes the Top-K inside the Full layer's candidate
pool; Reuse reads the Main KV and the latest Top-K.  [ZB] "把 KV Cache 压缩推到极致"
§2.3.2-§2.3.3 states the same modes and blocks: Encoder = 2 SWA layers + 3 blocks of
(Full, 5 x Reuse) at m = 2, one cache per block; Decoder = (Full, 3 x Reuse) + 4 blocks
of (Reindex, 3 x Reuse) at m = 1 over one cache, the Reindex layers choosing inside the
Decoder Full layer's pool ([ZB] §2.3.4).  The two SWA-only layers touch no global cache
and are outside the global branch; they are listed and skipped.

A decoding token at 0-based position p completes an entry of a cache with ratio m when
(p + 1) is a multiple of m; the entry pools the m newest latents of that cache's
source layer, at position m * j for entry j ([DF] §4.2; reading 4 of the design notes).
"""
from __future__ import annotations

import numpy as np

from . import block_topk, compress_pack, index_score, rope_table, sparse_attn


def layer_plan():
    """[(mode, cache)] for the 40 layers, 0-based; mode in swa / full / reindex / reuse."""
    plan = [("swa", None), ("swa", None)]
    for b in range(3):
        plan += [("full", "enc%d" % b)] + [("reuse", "enc%d" % b)] * 5
    plan += [("full", "dec")] + [("reuse", "dec")] * 3
    for _ in range(4):
        plan += [("reindex", "dec")] + [("reuse", "dec")] * 3
    return plan


CACHE_RATIO = {"enc0": 2, "enc1": 2, "enc2": 2, "dec": 1}


class SeqCaches:
    """One cache (main KV + indexer K) per source, for n_seq sequences of capacity cap
    entries each (sequence s owns rows s * cap ...)."""

    def __init__(self, n_seq, cap):
        self.n_seq, self.cap = n_seq, cap
        self.kv = {c: np.zeros((n_seq * cap, 288), np.uint8) for c in CACHE_RATIO}
        self.ix = {c: np.zeros((n_seq * cap, 68), np.uint8) for c in CACHE_RATIO}
        self.n = {c: 0 for c in CACHE_RATIO}


def decode_token(caches, p, new_latents, params, layer_inputs, K=512, M=2048):
    """Runs one decoding token at position p through every CSA2 layer.

    new_latents[c]: bf16 bits [n_seq, m_c, 512], the m_c newest latents of cache c's
    source (used only when the token completes an entry).  params[c] = (pool_w [m, 512],
    w_idx bf16 [128, 512]).  layer_inputs[l]: dict with q (bf16 [n_seq, 64, 512]), swa
    (bf16 [n_seq * 128, 512]), swa_len (int32 [n_seq]) and, for Full / Reindex layers,
    q_idx (bf16 [n_seq, 32, 128]) and head_w (fp32 [n_seq, 32]).
    Returns {layer: (out [n_seq, 64, 512], lse [n_seq, 64])} for the CSA2 layers."""
    n_seq, cap = caches.n_seq, caches.cap
    base = np.arange(n_seq, dtype=np.int64) * cap
    swa_start = np.arange(n_seq, dtype=np.int64) * 128
    outs = {}
    pool = topk = None
    for layer, (mode, c) in enumerate(layer_plan()):
        if mode == "swa":
            continue
        inp = layer_inputs[layer]
        m = CACHE_RATIO[c]
        if mode == "full":
            if (p + 1) % m == 0:  # this token completes entry j of cache c
                j = caches.n[c]
                pool_w, w_idx = params[c]
                kv, ix = compress_pack(new_latents[c].reshape(n_seq * m, 512), m, pool_w,
                                       rope_table(np.full(n_seq, m * j, np.int64)), w_idx)
                caches.kv[c][base + j] = kv
                caches.ix[c][base + j] = ix
                caches.n[c] = j + 1
            n = caches.n[c]
            nvis = np.full(n_seq, n, np.int32)
            scores = index_score(inp["q_idx"], inp["head_w"], caches.ix[c], base, nvis, n)
            pool, topk = block_topk(scores, nvis, K=K, M=M)
        elif mode == "reindex":
            n = caches.n[c]
            nvis = np.full(n_seq, n, np.int32)
            scores = index_score(inp["q_idx"], inp["head_w"], caches.ix[c], base, nvis, 8 * M,
                                 pool_blocks=pool)
            _, topk = block_topk(scores, nvis, K=K, M=M, pool_blocks=pool)
        outs[layer] = sparse_attn(inp["q"], caches.kv[c], base, topk, inp["swa"], swa_start, inp["swa_len"])
    return outs
