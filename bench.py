"""Benchmark: decode queries/s through the CSA2 global branch at 1M context on one MI355X.

Workload (decode_1m_b4_m2): 4 sequences x 1,048,576 tokens compressed at m = 2 into
524,288 FP4 entries each (main KV 288 B + indexer K 68 B per entry), 4 decode queries,
one Full layer.  One step runs the whole hot path once for the batch:
  append of each sequence's newest entry into its cache row (pool 2 latents, RoPE, FP4 +
  MXFP4 pack) fused with index_score over all 524,288 entries per query (+ block maxima),
  one launch (csa2_append_index_score: the append runs beside the scan, and the tile
  holding the new entry is scored once the entry is written)
  -> block_topk (top-2048 blocks of 8 -> pool -> Top-512)
  -> sparse_attn (64 heads over the 512 selected entries + 128 window rows).
Inputs are resident in HBM before timing starts.  The batch exists in NCOPY distinct
copies used round-robin so that the 142.6 MB indexer working set of a step is not served
from the 256 MB Infinity Cache left warm by the previous step.

Prints one JSON line (rank 0, N = 1).  `value` is queries/s over exactly K steps, replayed
from a HIP graph that holds NCOPY consecutive steps (one per batch copy), as a decoding
token's layers run inside one graph; `ms_per_step_one_step_graphs` is the same K steps with
one graph launch per step; `stages_us` times each stage of the step alone and
`replaced_stages_us` the separate append and scan launches the fused stage replaces;
`roofline` prices the dominant kernel (the fused append + scan) at 68 algorithmic bytes
per scored entry against 8 TB/s, timed with HIP events on the launch stream;
`roofline_step` prices the whole step (scan, selection, attention: 68 B per scored entry plus
each query's attention bytes) and `roofline_step_128k` the 128K batch-16 step (Full + Reindex
+ 3 Reuse) the same way; `step_us_p10_p50_p90` is the spread of single graph replays;
`ms_per_step_5_copies` repeats the step over 5 batch copies (a cache control);
`peaks_measured` holds a 1 GiB device copy and a bf16 GEMM beside the published peaks;
`cpu_baseline` times the oracle (plain C) on the same per-query work, one instance per host
thread, with the one-thread figure, the thread count and the CPU model.  `roofline.traffic`
is the HBM bytes per launch of that kernel from rocprofv3 FETCH_SIZE + WRITE_SIZE counters
(each scaled by what the counter reads for a torch copy of known size), read from
profiles/append_index_traffic.json and reported only while the kernel's sources still hash
to the ones those counters measured.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "decode_1m_b4_m2"
NCOPY = 3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=60)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--tokens", type=int, default=1048576, help="tokens per sequence")
    p.add_argument("--no-secondary", action="store_true", help="skip the other seeded workloads")
    p.add_argument("--no-peaks", action="store_true", help="skip the copy / GEMM peak measurements")
    p.add_argument("--no-control", action="store_true", help="skip the 5-copy cache control")
    p.add_argument("--no-handoff", action="store_true",
                   help="the selection takes its own first pass instead of the fused launch counting it")
    p.add_argument("--calibration-copy-mib", type=int, default=0,
                   help="run one device copy of this many MiB before timing (counter calibration)")
    return p.parse_args()


def make_batch(csa2, torch, copy_id, n_seq, tokens, m, chunk_tokens=1 << 19, extra_layers=0):
    """Builds one batch copy on the GPU: latents drawn with torch's seeded generator (N(0,1),
    RMS-normalised, bf16), packed into the caches by csa2_compress_pack.  extra_layers > 0
    adds a Reindex layer (fresh q_idx ~ N(0,1), head weights, q, window rows) and
    extra_layers - 1 Reuse layers (fresh q and window rows)."""
    dev = torch.device("cuda")
    n = tokens // m
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + copy_id)
    z = torch.randn((m, 512), generator=gen, device=dev, dtype=torch.float32)
    pool_w = torch.nn.functional.softplus(z).contiguous()
    w_idx = (torch.randn((128, 512), generator=gen, device=dev) / 512 ** 0.5).to(torch.bfloat16).contiguous()
    tile = csa2.IDX_TILE_ENTRIES
    assert n % tile == 0 and chunk_tokens % (tile * m) == 0  # sequences and chunks start indexer tiles
    kv = torch.empty((n_seq * n, 288), dtype=torch.uint8, device=dev)
    ix = torch.empty((n_seq * n // tile, csa2.IDX_TILE_BYTES), dtype=torch.uint8, device=dev)
    last_lat = torch.empty((n_seq, m, 512), dtype=torch.bfloat16, device=dev)
    pos_all = np.arange(n, dtype=np.int64) * m
    cs_all = csa2.rope_table(pos_all).to(dev)
    for s in range(n_seq):
        for t0 in range(0, tokens, chunk_tokens):
            tl = min(chunk_tokens, tokens - t0)
            x = torch.randn((tl, 512), generator=gen, device=dev, dtype=torch.float32)
            x = x / torch.sqrt(torch.mean(x * x, dim=1, keepdim=True) + 1e-6)
            xb = x.to(torch.bfloat16).contiguous()
            e0 = t0 // m
            csa2.compress_pack(xb, m, pool_w, cs_all[e0:e0 + tl // m], w_idx,
                               kv_out=kv[s * n + e0:], idx_out=ix[(s * n + e0) // tile:])
            if t0 + tl == tokens:
                last_lat[s] = xb[-m:]
        del x, xb
    q_idx = (torch.randn((n_seq, 32, 128), generator=gen, device=dev) / 128 ** 0.5).to(torch.bfloat16)
    head_w = torch.randn((n_seq, 32), generator=gen, device=dev) / 32 ** 0.5
    q = torch.randn((n_seq, 64, 512), generator=gen, device=dev).to(torch.bfloat16)
    sw = torch.randn((n_seq * 128, 512), generator=gen, device=dev)
    swa = (sw / torch.sqrt(torch.mean(sw * sw, dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16)
    layers = []
    for li in range(extra_layers):
        q_l = torch.randn((n_seq, 64, 512), generator=gen, device=dev).to(torch.bfloat16).contiguous()
        sw = torch.randn((n_seq * 128, 512), generator=gen, device=dev)
        sw_l = (sw / torch.sqrt(torch.mean(sw * sw, dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16).contiguous()
        lay = dict(q=q_l, swa=sw_l)
        if li == 0:
            lay["q_idx"] = torch.randn((n_seq, 32, 128), generator=gen, device=dev).to(torch.bfloat16).contiguous()
            lay["head_w"] = (torch.randn((n_seq, 32), generator=gen, device=dev) / 32 ** 0.5).contiguous()
        layers.append(lay)
    return dict(kv=kv, ix=ix, last_lat=last_lat.contiguous(), pool_w=pool_w, w_idx=w_idx,
                cs_last=cs_all[n - 1:n].contiguous(), q_idx=q_idx.contiguous(), head_w=head_w.contiguous(),
                q=q.contiguous(), swa=swa.contiguous(), layers=layers)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_threads():
    """Host threads the all-core leg may use: the process's CPU affinity, capped by the
    thread budget the environment sets (OMP_NUM_THREADS) when there is one."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(n_entries, n_q):
    """The oracle as it stands (plain C behind ctypes, which releases the interpreter lock
    during each call), on full 1M-context decode queries: each query is the whole path
    (compress of the newest entry, scoring of every entry, block/Top-K selection, attention).
    Timed on one host thread for n_q queries, then with one oracle instance per host thread
    on independent queries (two per thread)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from fp4_kv_cache_csa2_amd import synth
    kv, ix = synth.random_caches(99, n_entries)
    ci = synth.compress_inputs(98, 1, 2)
    d = synth.query_inputs(97, 1)
    cs = oracle.rope_table(np.array([2 * (n_entries - 1)], np.int64))

    def one_query(_=None):
        oracle.compress_pack(ci.latent, 2, ci.pool_w, cs, ci.w_idx)
        s = oracle.index_score(d.q_idx, d.head_w, ix, [0], [n_entries], n_entries)
        _, tk = oracle.block_topk(s, [n_entries])
        oracle.sparse_attn(d.q, kv, [0], tk, d.swa, d.swa_start, d.swa_len)

    t0 = time.perf_counter()
    for _ in range(n_q):
        one_query()
    dt1 = time.perf_counter() - t0
    threads = _host_threads()
    n_all = 2 * threads
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(one_query, range(n_all)))
        dt_all = time.perf_counter() - t0
    return {"value": round(n_all / dt_all, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_all} decode queries x {n_entries} entries, one oracle instance per host thread "
                      f"({threads} threads, {dt_all:.1f} s wall); each query the full path: compress of the newest "
                      f"entry, index over every entry, block/Top-K selection, attention",
            "single_thread": {"value": round(n_q / dt1, 3), "unit": "queries/s", "cores": 1,
                              "sample": f"{n_q} queries, {dt1:.1f} s on one host thread"},
            "cpu_model": _cpu_model(), "nproc": os.cpu_count()}


def measure_peaks(torch):
    """What this GPU reaches on plain library work, beside the published peaks: a device copy
    of 1 GiB (read + write bytes per second) and a bf16 8192^3 matrix product (hipBLASLt
    through torch), each the median of 5 timed repetitions with HIP events."""
    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    nb = 1 << 30
    src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    n = 8192
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_GBps": round(2 * nb / t_copy / 1e9, 1), "copy_bytes": nb,
            "bf16_gemm_TFLOPs": round(2 * n ** 3 / t_mm / 1e12, 1), "gemm_shape": [n, n, n],
            "published": {"hbm_GBps": HBM_PEAK_GBS, "bf16_dense_TFLOPs": 2500.0}}


class Decode1M:
    """Device state for a decode workload: one Full layer (compress the newest entry, score,
    select, attend), optionally followed by a Reindex layer (re-score the pool, select inside
    it, attend) and Reuse layers (attend with the Reindex indices)."""

    def __init__(self, torch, csa2, tokens, n_seq=4, m=2, K=512, M=2048, ncopy=NCOPY, extra_layers=0,
                 fp8_window=False, fp4q=False, hisa=False, handoff=True):
        self.torch, self.csa2 = torch, csa2
        # handoff (bf16 query, no HISA): the fused launch also counts the selection's first pass
        # into the selection workspace (csa2_append_index_score_sel) and the selection skips it
        # (csa2_block_topk_prebuilt)
        self.handoff = handoff and not (fp4q or hisa)
        self.fp8 = fp8_window
        self.fp4q = fp4q
        self.hisa = hisa
        self.n_seq, self.m, self.tokens, self.K, self.M, self.ncopy = n_seq, m, tokens, K, M, ncopy
        self.extra = extra_layers
        n = self.n = tokens // m
        dev = torch.device("cuda")
        print(f"[bench] building {ncopy} batch copies of {n_seq} x {tokens} tokens (m={m})", file=sys.stderr,
              flush=True)
        self.copies = [make_batch(csa2, torch, c, n_seq, tokens, m, extra_layers=extra_layers) for c in range(ncopy)]
        torch.cuda.synchronize()
        self.q_base = torch.arange(n_seq, dtype=torch.int64, device=dev) * n
        self.q_nvis = torch.full((n_seq,), n, dtype=torch.int32, device=dev)
        self.swa_start = torch.arange(n_seq, dtype=torch.int64, device=dev) * 128
        self.swa_len = torch.full((n_seq,), 128, dtype=torch.int32, device=dev)
        self.scores = torch.empty((n_seq, n), dtype=torch.float32, device=dev)
        self.bmax = torch.empty((n_seq, (n + 7) // 8), dtype=torch.float32, device=dev)
        self.pool = torch.empty((n_seq, M), dtype=torch.int32, device=dev)
        self.topk = torch.empty((n_seq, K), dtype=torch.int32, device=dev)
        self.out = torch.empty((n_seq, 64, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((n_seq, 64), dtype=torch.float32, device=dev)
        # the selection workspace starts zeroed and every call leaves its histogram zeroed
        self.ws_sel = torch.zeros(max(4, csa2.block_topk_workspace(n_seq, n, M, K)), dtype=torch.uint8, device=dev)
        # the fused stage timed on its own counts into this region, which no selection reads
        self.ws_hist_alone = torch.zeros(n_seq * 4096 * 4, dtype=torch.uint8, device=dev)
        self.ws_att = torch.empty(max(1, csa2.sparse_attn_workspace(n_seq, K)), dtype=torch.uint8, device=dev)
        # the step appends each sequence's newest entry into its cache slot, the last visible row
        # (the batch's caches were packed from the same latents, so every replay rewrites the same
        # bytes)
        self.new_rows = (self.q_base + (n - 1)).contiguous()
        self.cs_new = [c["cs_last"].expand(n_seq, 64).contiguous() for c in self.copies]
        if extra_layers:
            self.scores_r = torch.empty((n_seq, 8 * M), dtype=torch.float32, device=dev)
            self.topk_r = torch.empty((n_seq, K), dtype=torch.int32, device=dev)
        # the stages of one step: the append fused with the Full layer's scan (with HISA, the
        # append, the newest block's mean and the scan of the block means in one launch),
        # selection, attention, then the Reindex and Reuse layers
        self.step_stages = ([FUSED_HISA] if hisa else [FUSED]) + [2, 3] + (
            list(range(4, 6 + extra_layers)) if extra_layers else [])
        if fp4q:  # the fused launch packs the layer's bf16 indexer query into MXFP4 records itself
            # (the buffer serves the separate packer + scan, stage 1)
            self.q_fp4 = torch.empty((n_seq, 32, 68), dtype=torch.uint8, device=dev)
        if hisa:
            # HISA: every batch copy keeps the block-mean records of its caches; a step appends
            # the newest entry, re-packs its block's mean and scores the block means (one
            # launch), keeps the top-M blocks, then scores their entries and takes the Top-K
            # inside them
            self.nbw = (n + 7) // 8
            self.mbase = (torch.arange(n_seq, dtype=torch.int64, device=dev) * self.nbw).contiguous()
            self.s_blk = torch.empty((n_seq, self.nbw), dtype=torch.float32, device=dev)
            self.scores_c = torch.empty((n_seq, 8 * M), dtype=torch.float32, device=dev)
            for c in self.copies:
                c["means"] = torch.empty((csa2.idx_tiles_for(n_seq * self.nbw), csa2.IDX_TILE_BYTES),
                                         dtype=torch.uint8, device=dev)
                csa2.block_mean_pack(c["ix"], self.q_base, self.q_nvis, self.nbw, c["means"], self.mbase)
            torch.cuda.synchronize()
        if fp8_window:
            # per-sequence FP8 window rings of 128 rows; each step packs the newest token's
            # row into its slot, then attends over the ring (oldest row first)
            slot = torch.arange(n_seq, dtype=torch.int64, device=dev) * 128 + (tokens - 1) % 128
            self.ring_slot = slot.contiguous()
            self.ring_start = (torch.arange(n_seq, dtype=torch.int64, device=dev) * 128 + tokens % 128).contiguous()
            for ci, c in enumerate(self.copies):
                c["swa8"] = csa2.swa_pack_fp8(c["swa"])
                gen = torch.Generator(device=dev)
                gen.manual_seed(2000 + ci)
                x = torch.randn((n_seq, 512), generator=gen, device=dev)
                c["new_row"] = (x / torch.sqrt(torch.mean(x * x, dim=1, keepdim=True) + 1e-6)).to(
                    torch.bfloat16).contiguous()
            torch.cuda.synchronize()

    def add_copies(self, total):
        """More batch copies (the same recipe, further seeds) up to `total`, for the cache control."""
        torch, csa2 = self.torch, self.csa2
        while len(self.copies) < total:
            c = make_batch(csa2, torch, len(self.copies), self.n_seq, self.tokens, self.m, extra_layers=self.extra)
            self.copies.append(c)
            self.cs_new.append(c["cs_last"].expand(self.n_seq, 64).contiguous())
        torch.cuda.synchronize()

    def run_stage(self, ci, st, alone=False):
        """One stage of the step for batch copy ci, on torch's current stream (alone: the fused
        stage timed by itself, counting into a region no selection reads)."""
        c, csa2, n = self.copies[ci], self.csa2, self.n
        if st == FUSED:  # append each sequence's newest entry and score every entry, one launch
            # (with the MXFP4 query, the launch packs the bf16 query itself)
            sel_ws = (self.ws_hist_alone if alone else self.ws_sel) if self.handoff else None
            csa2.append_index_score(c["last_lat"].view(self.n_seq * self.m, 512), self.m, c["pool_w"],
                                    self.cs_new[ci], c["w_idx"], c["kv"], c["ix"], c["q_idx"], c["head_w"],
                                    self.q_base, self.q_nvis, n, scores=self.scores, block_max=self.bmax,
                                    pack_q=self.fp4q, sel_workspace=sel_ws)
        elif st == FUSED_HISA:  # append, re-pack the newest block's mean, score the block means
            csa2.append_mean_index_score(c["last_lat"].view(self.n_seq * self.m, 512), self.m, c["pool_w"],
                                         self.cs_new[ci], c["w_idx"], c["kv"], c["ix"], c["means"], self.mbase,
                                         c["q_idx"], c["head_w"], self.q_base, self.q_nvis, self.nbw,
                                         scores=self.s_blk)
        elif st == 0:  # append the newest entry of every sequence, from its m latest latents
            csa2.compress_append(c["last_lat"].view(self.n_seq * self.m, 512), self.m, c["pool_w"], self.cs_new[ci],
                                 c["w_idx"], self.new_rows, c["kv"], c["ix"])
        elif st == 2 and self.hisa:
            csa2.block_topk(None, self.q_nvis, K=self.K, M=self.M, block_max=self.s_blk, pool_out=self.pool,
                            want_topk=False, workspace=self.ws_sel)
            csa2.index_score(c["q_idx"], c["head_w"], c["ix"], self.q_base, self.q_nvis, 8 * self.M,
                             pool_blocks=self.pool, scores=self.scores_c)
            csa2.block_topk(self.scores_c, self.q_nvis, K=self.K, pool_blocks=self.pool, topk_out=self.topk,
                            workspace=self.ws_sel)
        elif st == 1 and self.fp4q:
            csa2.quantize_q_mxfp4(c["q_idx"], out=self.q_fp4)
            csa2.index_score_fp4q(self.q_fp4, c["head_w"], c["ix"], self.q_base, self.q_nvis, n, scores=self.scores,
                                  block_max=self.bmax)
        elif st == 1:
            csa2.index_score(c["q_idx"], c["head_w"], c["ix"], self.q_base, self.q_nvis, n, scores=self.scores,
                             block_max=self.bmax)
        elif st == 2:
            csa2.block_topk(self.scores, self.q_nvis, K=self.K, M=self.M, block_max=self.bmax, pool_out=self.pool,
                            topk_out=self.topk, workspace=self.ws_sel, hist_ready=self.handoff)
        elif st == SEL_FULL:  # the selection with its own first pass (valid on its own)
            csa2.block_topk(self.scores, self.q_nvis, K=self.K, M=self.M, block_max=self.bmax, pool_out=self.pool,
                            topk_out=self.topk, workspace=self.ws_sel)
        elif st == 3 and self.fp8:
            csa2.swa_pack_fp8(c["new_row"], out=c["swa8"], dst_rows=self.ring_slot)
            csa2.sparse_attn_swa_fp8(c["q"], c["kv"], self.q_base, self.topk, c["swa8"], self.ring_start,
                                     self.swa_len, swa_ring=128, out=self.out, lse=self.lse, workspace=self.ws_att)
        elif st == 3:
            csa2.sparse_attn(c["q"], c["kv"], self.q_base, self.topk, c["swa"], self.swa_start, self.swa_len,
                             out=self.out, lse=self.lse, workspace=self.ws_att)
        elif st == 4:  # Reindex layer: re-score the pool with its own indexer query
            lay = c["layers"][0]
            csa2.index_score(lay["q_idx"], lay["head_w"], c["ix"], self.q_base, self.q_nvis, 8 * self.M,
                             pool_blocks=self.pool, scores=self.scores_r)
        elif st == 5:
            csa2.block_topk(self.scores_r, self.q_nvis, K=self.K, pool_blocks=self.pool, topk_out=self.topk_r,
                            workspace=self.ws_sel)
        else:  # Reindex attention (st 6) and Reuse attention (st 7 ..) on the Reindex indices
            lay = c["layers"][st - 6]
            csa2.sparse_attn(lay["q"], c["kv"], self.q_base, self.topk_r, lay["swa"], self.swa_start, self.swa_len,
                             out=self.out, lse=self.lse, workspace=self.ws_att)


def attn_bytes_per_query(K=512, swa=128):
    """Algorithmic bytes of one query's attention: the K gathered 288-byte entries, the window
    rows (1 KiB of bf16 each), the query (64 x 512 bf16) and the output (64 x 512 fp32)."""
    return K * 288 + swa * 1024 + 64 * 512 * 2 + 64 * 512 * 4


def step_bytes(n_seq, n_entries, reindex_pool=0, attn_layers=1):
    """Algorithmic bytes of a decode step: the indexer scan (68 B per visible entry per query),
    a Reindex layer's pool (68 B per candidate), and each attention layer."""
    return n_seq * (n_entries * 68 + reindex_pool * 68 + attn_layers * attn_bytes_per_query())


def roofline(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_step": int(nbytes), "us_per_step": round(us, 2)}


FUSED = -1  # the stage that appends and scores in one launch (csa2_append_index_score)
FUSED_HISA = -2  # HISA's append + newest block mean + scan of the means (csa2_append_mean_index_score)
SEL_FULL = -3  # the selection with its own first pass (the step's selection skips it after the fused stage)
STAGE_NAMES = {FUSED: "append_index_score", FUSED_HISA: "append_mean_index_score", 0: "compress_newest",
               1: "index_score", 2: "block_topk", 3: "sparse_attn"}


def time_decode(torch, csa2, tokens, n_seq, m, extra_layers=0, steps=20, warmup=3, fp8_window=False, fp4q=False,
                hisa=False):
    """Whole-step throughput of a secondary decode workload: one HIP graph per batch copy
    holding every stage of the step, replayed `steps` times between two synchronisations."""
    wl = Decode1M(torch, csa2, tokens, n_seq=n_seq, m=m, extra_layers=extra_layers, fp8_window=fp8_window, fp4q=fp4q,
                  hisa=hisa)
    for i in range(warmup):
        for st in wl.step_stages:
            wl.run_stage(i % NCOPY, st)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    graphs = []
    for ci in range(NCOPY):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for st in wl.step_stages:
                wl.run_stage(ci, st)
        graphs.append(g)
    for i in range(2 * NCOPY):
        graphs[i % NCOPY].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % NCOPY].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = wall * 1e6 / steps
    res = {"queries_per_s": round(n_seq * steps / wall, 1), "us_per_step": round(us, 2),
           "sequences": n_seq, "tokens_per_sequence": tokens, "compress_ratio": m, "entries_per_sequence": wl.n,
           "layers": "Full" + (f" + Reindex + {extra_layers - 1} Reuse" if extra_layers else ""),
           "window": "FP8 rings (append + attend)" if fp8_window else "bf16",
           "indexer_query": "MXFP4 (packed inside the fused launch)" if fp4q else "bf16"}
    if extra_layers:
        # each stage of the step alone: HIP events around graphs of back-to-back launches
        names = {FUSED: "append_index_score", 2: "block_topk", 3: "sparse_attn_full", 4: "reindex_index_score",
                 5: "reindex_block_topk", 6: "sparse_attn_reindex"}
        # (with the handoff the Full selection reads the counts of the fused launch before it:
        # it is timed as a graph of both minus one of the fused launch alone)
        res["stages_us"] = {}
        us_of = {}
        for st in wl.step_stages:
            reps = 4 * NCOPY
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for r in range(reps):
                    if st == 2 and wl.handoff:
                        wl.run_stage(r % NCOPY, FUSED)
                    wl.run_stage(r % NCOPY, st, alone=True)
            g.replay()
            torch.cuda.synchronize()
            samples = []
            for _ in range(7):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                samples.append(a.elapsed_time(b) * 1e3 / reps)
            us_of[st] = float(np.median(samples))
            if st == 2 and wl.handoff:
                us_of[st] -= us_of[FUSED]
            res["stages_us"][names.get(st, f"sparse_attn_reuse{st - 6}")] = round(us_of[st], 2)
            del g
    if not hisa and not fp8_window:
        # the whole step against the HBM roofline: Full scan, Reindex pool, every attention layer
        nbytes = step_bytes(n_seq, wl.n, reindex_pool=8 * wl.M if extra_layers else 0, attn_layers=1 + extra_layers)
        res["roofline_step"] = roofline(nbytes, us)
    if hisa:
        # recall of the exact Top-K (the Full layer's, over every entry) by HISA's Top-K, on the
        # last replayed copy's inputs
        ci = (steps - 1) % NCOPY
        hisa_topk = wl.topk.clone()
        c = wl.copies[ci]
        csa2.index_score(c["q_idx"], c["head_w"], c["ix"], wl.q_base, wl.q_nvis, wl.n, scores=wl.scores,
                         block_max=wl.bmax)
        csa2.block_topk(wl.scores, wl.q_nvis, K=wl.K, M=wl.M, block_max=wl.bmax, pool_out=wl.pool,
                        topk_out=wl.topk, workspace=wl.ws_sel)
        torch.cuda.synchronize()
        a, b = hisa_topk.cpu().numpy(), wl.topk.cpu().numpy()
        rec = [len(np.intersect1d(a[t][a[t] >= 0], b[t][b[t] >= 0])) / max(1, int((b[t] >= 0).sum()))
               for t in range(n_seq)]
        res["layers"] = "Full with HISA selection (block means -> top-2048 blocks -> Top-512 inside)"
        res["recall_of_exact_topk"] = round(float(np.mean(rec)), 4)
    del graphs, wl
    torch.cuda.empty_cache()
    return res


def time_prefill(torch, csa2, hist_tokens=65536, chunk=4096, m=2, reps=10):
    """The chunked-prefill workload, one launch per stage timed with HIP events: compress the
    chunk's 2048 new entries from latents, causal scoring of 4096 queries over <= 34816
    entries, per-query Top-512, attention for every query.  The history caches are drawn
    directly (uniform FP4 codes, scale bytes of the synthetic range)."""
    from fp4_kv_cache_csa2_amd import synth
    dev = torch.device("cuda")
    hist = hist_tokens // m
    n = hist + chunk // m
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    kv = torch.randint(0, 256, (n, 288), dtype=torch.uint8, device=dev, generator=g)
    kv[:, 256:] = 0x30
    assert hist % csa2.IDX_TILE_ENTRIES == 0  # the chunk's new entries start an indexer tile
    ix = torch.randint(0, 256, (csa2.idx_tiles_for(n), csa2.IDX_TILE_BYTES), dtype=torch.uint8, device=dev,
                       generator=g)
    ix[:, 2048:] = 126  # every entry's four E8M0 scale bytes
    nvis = torch.from_numpy(synth.prefill_nvis(hist_tokens, chunk, m)).to(dev)
    q_idx = (torch.randn((chunk, 32, 128), device=dev, generator=g) / 128 ** 0.5).to(torch.bfloat16)
    head_w = torch.randn((chunk, 32), device=dev, generator=g) / 32 ** 0.5
    q = torch.randn((chunk, 64, 512), device=dev, generator=g).to(torch.bfloat16)
    sw = torch.randn((chunk + 127, 512), device=dev, generator=g)
    swa = (sw / torch.sqrt(torch.mean(sw * sw, dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16)
    base = torch.zeros(chunk, dtype=torch.int64, device=dev)
    swa_start = torch.arange(chunk, dtype=torch.int64, device=dev)
    swa_len = torch.full((chunk,), 128, dtype=torch.int32, device=dev)
    x = torch.randn((chunk, 512), device=dev, generator=g)
    lat = (x / torch.sqrt(torch.mean(x * x, dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16)
    pool_w = torch.nn.functional.softplus(torch.randn((m, 512), device=dev, generator=g)).contiguous()
    w_idx = (torch.randn((128, 512), device=dev, generator=g) / 512 ** 0.5).to(torch.bfloat16)
    cs = csa2.rope_table(np.arange(hist, n, dtype=np.int64) * m).to(dev)
    scores = torch.empty((chunk, n), dtype=torch.float32, device=dev)
    topk = torch.empty((chunk, 512), dtype=torch.int32, device=dev)
    out = torch.empty((chunk, 64, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((chunk, 64), dtype=torch.float32, device=dev)
    ws = torch.zeros(csa2.block_topk_workspace(chunk, n, 2048, 512), dtype=torch.uint8, device=dev)
    wsa = torch.empty(max(16, csa2.sparse_attn_workspace(chunk, 512)), dtype=torch.uint8, device=dev)
    stages = {
        "compress_2048_entries": lambda: csa2.compress_pack(lat, m, pool_w, cs, w_idx, kv_out=kv[hist:],
                                                           idx_out=ix[hist // csa2.IDX_TILE_ENTRIES:]),
        "index_4096_queries": lambda: csa2.index_score(q_idx, head_w, ix, base, nvis, n, scores=scores,
                                                       want_block_max=False),
        "select_4096_queries": lambda: csa2.block_topk(scores, nvis, want_pool=False, topk_out=topk, workspace=ws),
        "attn_4096_queries": lambda: csa2.sparse_attn(q, kv, base, topk, swa, swa_start, swa_len, out=out,
                                                      lse=lse, workspace=wsa),
        # the same scoring with the indexer query packed to MXFP4 (FP4 x FP4 block-scaled MFMA)
        "pack_q_mxfp4": lambda: csa2.quantize_q_mxfp4(q_idx, out=q_fp4),
        "index_4096_queries_fp4q": lambda: csa2.index_score_fp4q(q_fp4, head_w, ix, base, nvis, n, scores=scores,
                                                                 want_block_max=False),
    }
    q_fp4 = torch.empty((chunk, 32, 68), dtype=torch.uint8, device=dev)
    ms = {}
    for name, fn in stages.items():
        fn()
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms[name] = round(a.elapsed_time(b) / reps, 4)
    flops = 2.0 * 32 * 128 * float(nvis.sum().item())
    bf16_path = ("compress_2048_entries", "index_4096_queries", "select_4096_queries", "attn_4096_queries")
    fp4_path = ("compress_2048_entries", "pack_q_mxfp4", "index_4096_queries_fp4q", "select_4096_queries",
                "attn_4096_queries")
    t_b, t_f = ms["index_4096_queries"] * 1e-3, ms["index_4096_queries_fp4q"] * 1e-3
    res = {"ms": ms, "total_ms": round(sum(ms[k] for k in bf16_path), 4),
           "total_ms_fp4q": round(sum(ms[k] for k in fp4_path), 4),
           "index_mfma": {"achieved_tflops": round(flops / t_b / 1e12, 1), "peak_tflops": 2500.0, "dtype": "bf16",
                          "frac": round(flops / t_b / 2.5e15, 4)},
           "index_mfma_fp4q": {"achieved_tflops": round(flops / t_f / 1e12, 1), "peak_tflops": 10100.0,
                               "dtype": "fp4", "frac": round(flops / t_f / 10.1e15, 4)}}
    del kv, ix, scores, out, ws, wsa
    torch.cuda.empty_cache()
    return res
def time_schedule(torch, csa2, tokens=1 << 20, n_seq=4, steps=10, warmup=2):
    """Decode tokens through all 38 CSA2 layers of the 40-layer stack at `tokens` context:
    3 Encoder caches (m = 2) and the Decoder cache (m = 1) packed from GPU-drawn latents,
    per-layer query / indexer query / head weights / window rows drawn once.  Two tokens
    are timed alternately, at positions `tokens` (the Decoder cache appends an entry) and
    `tokens + 1` (every cache appends), each as one HIP graph of the whole token."""
    from fp4_kv_cache_csa2_amd import schedule
    dev = torch.device("cuda")
    caps = {c: tokens // m + 2 for c, m in schedule.RATIO.items()}
    g = schedule.GlobalBranch(n_seq, caps)
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)

    def rms_bf16(shape):
        x = torch.randn(shape, generator=gen, device=dev)
        return (x / torch.sqrt(torch.mean(x * x, dim=-1, keepdim=True) + 1e-6)).to(torch.bfloat16).contiguous()

    print(f"[bench] schedule: packing 4 caches of {n_seq} x {tokens} tokens", file=sys.stderr, flush=True)
    chunk = 1 << 18
    for c, m in schedule.RATIO.items():
        pool_w = torch.nn.functional.softplus(torch.randn((m, 512), generator=gen, device=dev)).contiguous()
        w_idx = (torch.randn((128, 512), generator=gen, device=dev) / 512 ** 0.5).to(torch.bfloat16).contiguous()
        g.set_params(c, pool_w, w_idx)
        for t0 in range(0, tokens, chunk):
            g.fill(c, rms_bf16((n_seq, min(chunk, tokens - t0), 512)), first_entry=t0 // m)
    layers = schedule.csa2_layers()
    swa_start = (torch.arange(n_seq, dtype=torch.int64, device=dev) * 128).contiguous()
    swa_len = torch.full((n_seq,), 128, dtype=torch.int32, device=dev)
    inputs = {l: {"q": torch.randn((n_seq, 64, 512), generator=gen, device=dev).to(torch.bfloat16).contiguous(),
                  "swa": rms_bf16((n_seq * 128, 512)), "swa_start": swa_start, "swa_len": swa_len,
                  "q_idx": (torch.randn((n_seq, 32, 128), generator=gen, device=dev) / 128 ** 0.5).to(
                      torch.bfloat16).contiguous(),
                  "head_w": (torch.randn((n_seq, 32), generator=gen, device=dev) / 32 ** 0.5).contiguous()}
              for l in layers}
    new = {c: rms_bf16((n_seq * m, 512)) for c, m in schedule.RATIO.items()}
    outs = {l: torch.empty((n_seq, 64, 512), dtype=torch.float32, device=dev) for l in layers}
    positions = (tokens, tokens + 1)
    for _ in range(warmup):
        for p in positions:
            g.decode_token(p, new, inputs, outs)
    torch.cuda.synchronize()
    cap_stream = torch.cuda.Stream()
    graphs = []
    states = []
    for p in positions:
        st = g.token_state(p)  # the device state the graph of position p reads
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap_stream):
            g.decode_token(p, new, inputs, outs, state=st)
        graphs.append(gr)
        states.append(st)
    for gr in graphs:
        gr.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    res = {"tokens_per_s": round(n_seq * steps / wall, 1), "us_per_token_step": round(wall * 1e6 / steps, 1),
           "sequences": n_seq, "context_tokens": tokens,
           "caches": {c: {"m": m, "entries_per_sequence": tokens // m} for c, m in schedule.RATIO.items()},
           "layers": "40 (2 SWA-only skipped): 4 Full, 4 Reindex, 30 Reuse; 38 attention calls per token",
           "window": "bf16 rows, drawn once per layer"}
    del graphs, states, g, inputs, outs
    torch.cuda.empty_cache()
    return res


# the sources the fused append + scan kernel is built from
INDEX_SRCS = [os.path.join(ROOT, "fp4_kv_cache_csa2_amd", "csrc", f)
              for f in ("append_index.hip", "index_tiles.hpp", "index_common.hpp", "compress_few.hpp",
                        "block_mean.hpp", "csa2_device.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "append_index_traffic.json")


def index_source_sha():
    h = hashlib.sha256()
    for f in INDEX_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the fused append + scan kernel from the committed counter
    summary, or None when it is missing or was taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = index_source_sha()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha or rec.get("workload") != WORKLOAD:
        return None
    return int(rec["hbm_bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)
    import torch
    from fp4_kv_cache_csa2_amd import csa2

    torch.cuda.set_device(0)
    if args.calibration_copy_mib > 0:  # a plain copy of known size for counter calibration
        nb = args.calibration_copy_mib << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    peaks = None if args.no_peaks else measure_peaks(torch)
    wl = Decode1M(torch, csa2, args.tokens, handoff=not args.no_handoff)
    n_seq, m, tokens, n, K, M = wl.n_seq, wl.m, wl.tokens, wl.n, wl.K, wl.M
    step = wl.step_stages  # the fused append + scan, selection, attention
    # stages timed on their own: the step's, the selection with its own first pass, and the
    # two launches the fused stage replaces.  With the handoff the step's selection reads the
    # counts of the fused launch before it, so it is timed as a graph of both minus one of the
    # fused launch alone.
    timed = step + [SEL_FULL, 0, 1]
    alone = [st for st in timed if not (wl.handoff and st == 2)]
    run_stage = wl.run_stage
    for i in range(args.warmup):  # eager warm-up
        for st in timed:
            run_stage(i % NCOPY, st)
    torch.cuda.synchronize()
    # One HIP graph holds NCOPY consecutive steps, one per batch copy, as the layers of a
    # decoding token follow each other inside one graph: a replay runs NCOPY whole steps
    # back to back and the host's launch gap between replays is paid once per NCOPY steps.
    # A single-step graph per copy covers a remainder of steps and the per-step figure
    # below.
    cap = torch.cuda.Stream()
    multi_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi_graph, stream=cap):
        for ci in range(NCOPY):
            for st in step:
                run_stage(ci, st)
    step_graph = []
    for ci in range(NCOPY):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for st in step:
                run_stage(ci, st)
        step_graph.append(g)
    # per-stage graphs of back-to-back launches (rotating copies) for the stage timings
    reps = 4 * NCOPY
    stage_graph = []
    for st in alone:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for r in range(reps):
                run_stage(r % NCOPY, st, alone=True)
        stage_graph.append(g)
    pair_graph = None
    if wl.handoff:
        pair_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pair_graph, stream=cap):
            for r in range(reps):
                run_stage(r % NCOPY, FUSED)
                run_stage(r % NCOPY, 2)
        stage_graph.append(pair_graph)
    for i in range(2 * NCOPY):
        step_graph[i % NCOPY].replay()
    multi_graph.replay()
    for g in stage_graph:
        g.replay()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    # ---- timed region: exactly K steps (K // NCOPY multi-step replays, then the remaining
    # steps one graph each), synchronised on both sides
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps // NCOPY):
        multi_graph.replay()
    for i in range(args.steps % NCOPY):
        step_graph[i].replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = t1 - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = wall_s * 1e3 / args.steps
    value = n_seq * args.steps / wall_s

    # the same K steps with one graph per step (each replay pays the launch gap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_graph[i % NCOPY].replay()
    torch.cuda.synchronize()
    ms_single = (time.perf_counter() - t0) * 1e3 / args.steps

    # ---- stage timings: HIP events around graphs of back-to-back launches of one stage, the
    # median over 7 replays
    stage_samples = 7
    st_us = {}
    for st, g in zip(alone + (["pair"] if pair_graph is not None else []), stage_graph):
        samples = []
        for _ in range(stage_samples):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b) * 1e3 / reps)
        st_us[st] = float(np.median(samples))
    if pair_graph is not None:
        st_us[2] = st_us.pop("pair") - st_us[FUSED]
    # spread of the step time: HIP events around single replays of the multi-step graph
    per_step = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        multi_graph.replay()
        b.record()
        torch.cuda.synchronize()
        per_step.append(a.elapsed_time(b) * 1e3 / NCOPY)
    p10, p50, p90 = (float(np.percentile(per_step, q)) for q in (10, 50, 90))
    # cache control: the same step rotating over 5 batch copies (186 MB of caches each), so
    # any reuse of the 256 MB Infinity Cache between steps is further away; an equal time per
    # step means the 3-copy figure is not served from it
    ms_5 = None
    if not args.no_control:
        wl.add_copies(5)
        g5 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g5, stream=cap):
            for ci in range(5):
                for st in step:
                    run_stage(ci, st)
        g5.replay()
        torch.cuda.synchronize()
        reps5 = max(1, args.steps // 5)
        t0 = time.perf_counter()
        for _ in range(reps5):
            g5.replay()
        torch.cuda.synchronize()
        ms_5 = (time.perf_counter() - t0) * 1e3 / (5 * reps5)
        del g5
    # the dominant kernel: the fused append + scan; its algorithmic bytes are the scan's
    idx_us = st_us[FUSED]
    idx_bytes = n_seq * n * 68
    achieved = idx_bytes / (idx_us * 1e-6) / 1e9
    line = {
        "metric": "decode queries/s through CSA2 global branch at 1M ctx; % HBM roofline",
        "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD, "sequences": n_seq, "tokens_per_sequence": tokens,
                   "compress_ratio": m, "entries_per_sequence": n, "index_heads": 32, "index_dim": 128,
                   "pool_blocks": M, "block": 8, "topk": K, "heads": 64, "head_dim": 512,
                   "swa": 128, "batch_copies": NCOPY},
        "stages_us": {STAGE_NAMES[st]: round(float(st_us[st]), 2) for st in step},
        "first_pass_in_fused_launch": wl.handoff,
        "block_topk_with_first_pass_us": round(float(st_us[SEL_FULL]), 2),
        "replaced_stages_us": {STAGE_NAMES[st]: round(float(st_us[st]), 2) for st in (0, 1)},
        "gpu_ms_timed_region": round(gpu_ms, 4), "wall_s_timed_region": round(wall_s, 4),
        "steps_per_graph": NCOPY, "ms_per_step_one_step_graphs": round(ms_single, 4),
        "roofline": {"kernel": "append_index_score", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": idx_bytes},
        # the whole step (scan + selection + attention) against the same roofline
        "roofline_step": roofline(step_bytes(n_seq, n), ms_per_step * 1e3),
        "step_us_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)],
        "ms_per_step_5_copies": None if ms_5 is None else round(ms_5, 4),
        "peaks_measured": peaks,
    }
    if not args.no_secondary:
        # the other seeded workloads, each in its own graphs after the timed region above
        del step_graph, stage_graph, multi_graph, pair_graph, wl
        torch.cuda.empty_cache()
        print("[bench] secondary workloads", file=sys.stderr, flush=True)
        sec = {
            "decode_token_40layer_1m_b4": time_schedule(torch, csa2),
            "decode_1m_b4_m2_fp8_window": time_decode(torch, csa2, 1 << 20, 4, 2, fp8_window=True),
            "decode_1m_b4_m2_fp4q": time_decode(torch, csa2, 1 << 20, 4, 2, fp4q=True),
            "decode_1m_b4_m2_hisa": time_decode(torch, csa2, 1 << 20, 4, 2, hisa=True),
            "decode_128k_b16_m1": time_decode(torch, csa2, 131072, 16, 1, extra_layers=4),
            "decode_32k_b4_m1": time_decode(torch, csa2, 32768, 4, 1),
            "tiny_4k_b1_m2": time_decode(torch, csa2, 4096, 1, 2),
            "prefill_chunk4096_hist65536_m2": time_prefill(torch, csa2),
        }
        line["secondary"] = sec
        # the 128K batch-16 step (Full + Reindex + 3 Reuse) is the metric's other context
        line["roofline_step_128k"] = sec["decode_128k_b16_m1"]["roofline_step"]
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(n, n_seq)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
