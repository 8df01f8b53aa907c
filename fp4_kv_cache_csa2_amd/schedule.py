"""The CSA2 global branch over the whole 40-layer stack: one decoding token through every
CSA2 layer, issued as calls of the C ABI.

Layer plan ([DF] "4. 层维度(下):CSA2 与每 token 890 字节" §4.3; [ZB] "把 KV Cache 压缩推到极致"
§2.3.2-§2.3.4):
  - Encoder (layers 0-19, m = 2): 2 SWA-only layers, then 3 blocks of one Full layer and
    five Reuse layers; each block owns one cache.
  - Decoder (layers 20-39, m = 1, one cache): a Full layer and 3 Reuse layers, then 4
    blocks of one Reindex layer and 3 Reuse layers.  Reindex layers choose inside the
    candidate pool of the Decoder Full layer; Reuse layers attend with the latest Top-K.
The SWA-only layers touch no global cache and are not part of this path.

A token at position p completes an entry of a ratio-m cache when p + 1 is a multiple of
m; the Full layer of that cache then packs it from the m newest latents of its source, in
the same launch as its scan of the cache (csa2_append_index_score) when the new entry is
the newest visible one.
Device tensors only: every step runs in the library's kernels; the host decides which
call comes next from the plan and the position.
"""
from __future__ import annotations

import numpy as np
import torch

from . import csa2

RATIO = {"enc0": 2, "enc1": 2, "enc2": 2, "dec": 1}


def layer_plan():
    """[(mode, cache)] for layers 0..39; mode is 'swa', 'full', 'reindex' or 'reuse'."""
    enc = [("swa", None)] * 2
    for b in range(3):
        enc += [("full", f"enc{b}")] + [("reuse", f"enc{b}")] * 5
    dec = [("full", "dec")] + [("reuse", "dec")] * 3
    for _ in range(4):
        dec += [("reindex", "dec")] + [("reuse", "dec")] * 3
    return enc + dec


def csa2_layers():
    return [i for i, (mode, _) in enumerate(layer_plan()) if mode != "swa"]


class GlobalBranch:
    """Device state of the four global caches of n_seq sequences (capacity cap_c entries
    each; sequence s owns rows s * cap_c ...) and the scratch of one decoding token."""

    def __init__(self, n_seq, caps, K=512, M=2048, device="cuda"):
        # capacities are rounded up to whole tiles of 32 entries, so every sequence's first
        # indexer entry starts a tile of the indexer cache and bulk packing can write from there
        tile = csa2.IDX_TILE_ENTRIES
        caps = {c: (v + tile - 1) // tile * tile for c, v in caps.items()}
        self.n_seq, self.caps, self.K, self.M = n_seq, caps, K, M
        dev = self.dev = torch.device(device)
        self.kv = {c: torch.zeros((n_seq * caps[c], 288), dtype=torch.uint8, device=dev) for c in RATIO}
        self.ix = {c: torch.zeros((n_seq * caps[c] // tile, csa2.IDX_TILE_BYTES), dtype=torch.uint8, device=dev)
                   for c in RATIO}
        self.n = {c: 0 for c in RATIO}
        self.params = {}
        self.base = {c: torch.arange(n_seq, dtype=torch.int64, device=dev) * caps[c] for c in RATIO}
        width = max(caps.values())
        self.scores = torch.empty((n_seq, width), dtype=torch.float32, device=dev)
        self.bmax = torch.empty((n_seq, (width + 7) // 8), dtype=torch.float32, device=dev)
        self.scores_r = torch.empty((n_seq, 8 * M), dtype=torch.float32, device=dev)
        self.pool = torch.empty((n_seq, M), dtype=torch.int32, device=dev)
        self.topk = torch.empty((n_seq, K), dtype=torch.int32, device=dev)
        ws = max(csa2.block_topk_workspace(n_seq, width, M, K), csa2.block_topk_workspace(n_seq, 8 * M, M, K))
        self.ws_sel = torch.zeros(max(ws, 4), dtype=torch.uint8, device=dev)  # left zeroed by every call
        self.ws_att = torch.empty(max(csa2.sparse_attn_workspace(n_seq, K), 16), dtype=torch.uint8, device=dev)
        # the per-token device state of eager decoding, refilled in place for every token
        self._state = TokenState(self, None)

    def set_params(self, c, pool_w, w_idx):
        self.params[c] = (pool_w.contiguous(), w_idx.contiguous())

    def token_state(self, p):
        """The device tensors one token at position p reads (visible counts, the appended
        entries' RoPE rows and cache rows), owned by the caller: a HIP graph captured from
        decode_token(p, ..., state=s) stays valid while s lives."""
        return TokenState(self, p)

    def fill(self, c, latents, first_entry=0, chunk_tokens=1 << 19):
        """Bulk-pack entries first_entry .. of cache c from latents bf16 [n_seq, tokens, 512]."""
        m = RATIO[c]
        pool_w, w_idx = self.params[c]
        tokens = latents.shape[1]
        tile = csa2.IDX_TILE_ENTRIES
        assert first_entry % tile == 0 and chunk_tokens % (tile * m) == 0  # whole indexer tiles
        for s in range(self.n_seq):
            for t0 in range(0, tokens, chunk_tokens):
                tl = min(chunk_tokens, tokens - t0)
                e0 = first_entry + t0 // m
                pos = np.arange(e0, e0 + tl // m, dtype=np.int64) * m
                row = s * self.caps[c] + e0
                csa2.compress_pack(latents[s, t0:t0 + tl].contiguous(), m, pool_w, csa2.rope_table(pos).to(self.dev),
                                   w_idx, kv_out=self.kv[c][row:], idx_out=self.ix[c][row // tile:])
        self.n[c] = max(self.n[c], first_entry + tokens // m)

    def decode_token(self, p, new_latents, inputs, outs, lses=None, state=None):
        """One token at position p.  new_latents[c]: bf16 [n_seq * m_c, 512], the m_c newest
        latents of cache c's source (read only when p completes an entry).  inputs[l]: dict
        of device tensors q, swa, swa_start, swa_len, plus q_idx, head_w for Full and Reindex
        layers.  outs[l] / lses[l]: outputs of layer l.  state: token_state(p) for a call that
        is captured into a graph; by default the branch's own state tensors are refilled in
        place (no device memory is allocated per token)."""
        K, M = self.K, self.M
        for c in RATIO:  # the entries this token completes become visible
            m = RATIO[c]
            if (p + 1) % m == 0:
                self.n[c] = max(self.n[c], (p + 1) // m)
        if state is None:
            state = self._state
            state.refill(p)
        elif state.p != p or state.n != self.n:
            raise ValueError("state was made for another position")
        for layer, (mode, c) in enumerate(layer_plan()):
            if mode == "swa":
                continue
            inp = inputs[layer]
            if mode == "full":
                m = RATIO[c]
                j = (p + 1) // m - 1 if (p + 1) % m == 0 else None  # this token completes entry j of cache c
                n = self.n[c]
                nvis = state.nvis[c]
                if j is not None:
                    cs = state.rope[c]
                    pool_w, w_idx = self.params[c]
                fused = j is not None and j == n - 1
                if fused:
                    # the new entry is the newest visible one: append it and score in one launch,
                    # which also counts the selection's first pass into its workspace
                    csa2.append_index_score(new_latents[c], m, pool_w, cs, w_idx, self.kv[c], self.ix[c],
                                            inp["q_idx"], inp["head_w"], self.base[c], nvis, n,
                                            scores=self._row_view(n), block_max=self._bmax_view(n),
                                            sel_workspace=self.ws_sel)
                else:
                    if j is not None:
                        csa2.compress_append(new_latents[c], m, pool_w, cs, w_idx, state.rows[c], self.kv[c],
                                             self.ix[c])
                    csa2.index_score(inp["q_idx"], inp["head_w"], self.ix[c], self.base[c], nvis, n,
                                     scores=self._row_view(n), block_max=self._bmax_view(n))
                csa2.block_topk(self._row_view(n), nvis, K=K, M=M, block_max=self._bmax_view(n),
                                pool_out=self.pool, topk_out=self.topk, workspace=self.ws_sel, hist_ready=fused)
            elif mode == "reindex":
                nvis = state.nvis[c]
                csa2.index_score(inp["q_idx"], inp["head_w"], self.ix[c], self.base[c], nvis, 8 * M,
                                 pool_blocks=self.pool, scores=self.scores_r)
                csa2.block_topk(self.scores_r, nvis, K=K, pool_blocks=self.pool, topk_out=self.topk,
                                workspace=self.ws_sel)
            csa2.sparse_attn(inp["q"], self.kv[c], self.base[c], self.topk, inp["swa"], inp["swa_start"],
                             inp["swa_len"], out=outs[layer], lse=None if lses is None else lses[layer],
                             want_lse=lses is not None, workspace=self.ws_att)

    def _row_view(self, n):
        """A dense [n_seq, n] view of the score buffer (the kernels take rows of exactly `width`
        floats); a view allocates no device memory."""
        return self.scores.view(-1)[:self.n_seq * n].view(self.n_seq, n)

    def _bmax_view(self, n):
        nb = (n + 7) // 8
        return self.bmax.view(-1)[:self.n_seq * nb].view(self.n_seq, nb)


class TokenState:
    """Device tensors of one decoding token at position p: per cache the visible count of
    every sequence (int32 [n_seq]), and for the caches this token appends to, the new entry's
    RoPE row (fp32 [n_seq, 64]) and its cache row in every sequence (int64 [n_seq])."""

    def __init__(self, branch, p):
        self.b = branch
        ns, dev = branch.n_seq, branch.dev
        self.nvis = {c: torch.zeros(ns, dtype=torch.int32, device=dev) for c in RATIO}
        self.rope = {c: torch.zeros((ns, 64), dtype=torch.float32, device=dev) for c in RATIO}
        self.rows = {c: torch.zeros(ns, dtype=torch.int64, device=dev) for c in RATIO}
        self.p, self.n = None, None
        if p is not None:
            self.refill(p)

    def refill(self, p):
        """Rewrites the tensors in place for position p (stream-ordered after the launches
        that read their previous values), with the visible counts after p's appends."""
        b = self.b
        self.n = {c: max(b.n[c], (p + 1) // m) if (p + 1) % m == 0 else b.n[c] for c, m in RATIO.items()}
        for c, m in RATIO.items():
            self.nvis[c].fill_(self.n[c])
            if (p + 1) % m == 0:
                j = (p + 1) // m - 1
                self.rope[c].copy_(csa2.rope_table(np.full(b.n_seq, m * j, np.int64)))
                torch.add(b.base[c], j, out=self.rows[c])
        self.p = p
