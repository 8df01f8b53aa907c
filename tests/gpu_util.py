"""Helpers for the GPU parity tests: device transfer and the acceptance checks.

Acceptance (per output type): packed bytes bit-exact; block / entry selections identical
except members whose oracle score lies within 1e-4 relative of the M-th / K-th oracle
score (ties broken by the lower index on both sides); scores within 2e-5 of the row's
largest magnitude; attention outputs within 2e-3 max relative error, row-normwise
(max over query and head of ||o - r||_inf / ||r||_inf)."""
import numpy as np
import torch

from fp4_kv_cache_csa2_amd import layout

SEL_RTOL = 1e-4
ATTN_TOL = 2e-3
SCORE_TOL = 2e-5


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def dev_ix(rec):
    """A device indexer-K (or block-mean) cache in the kernels' tile layout holding the given
    68-byte records as entries 0 .. n - 1."""
    return dev(layout.records_to_tiles(rec))


def host_ix(t, n=None):
    """Entries 0 .. n - 1 (default: every slot) of a device tile-layout cache as 68-byte records."""
    a = host(t)
    return layout.tiles_to_records(a, a.shape[0] * layout.TILE_ENTRIES if n is None else n)


def ix_tensor(n, fill=0):
    """A device tile-layout cache with room for n entries, every byte set to fill."""
    tiles = (n + layout.TILE_ENTRIES - 1) // layout.TILE_ENTRIES
    return torch.full((tiles, layout.TILE_BYTES), fill, dtype=torch.uint8, device="cuda")


def check_scores(got, ref, nvis=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf pattern differs"
    for t in range(ref.shape[0]):
        r = ref[t][fin[t]]
        if r.size == 0:
            continue
        scale = max(np.max(np.abs(r)), 1e-30)
        err = np.max(np.abs(got[t][fin[t]] - r))
        assert err <= SCORE_TOL * scale, f"row {t}: score error {err:.3e} vs scale {scale:.3e}"


def check_selection(got_ids, ref_ids, key_of, what="topk"):
    """got/ref: ascending id lists padded with -1; key_of(ids) -> oracle ranking values."""
    got = np.asarray(got_ids)
    ref = np.asarray(ref_ids)
    g = got[got >= 0]
    r = ref[ref >= 0]
    assert np.all(np.diff(g) > 0), f"{what}: GPU output not strictly ascending"
    assert g.size == r.size, f"{what}: count {g.size} vs {r.size}"
    if np.array_equal(g, r):
        return 0
    kv = key_of(r)
    kth = np.min(kv)
    scale = max(abs(kth), 1e-6 * np.max(np.abs(kv)), 1e-30)
    extra = np.setdiff1d(g, r)
    missing = np.setdiff1d(r, g)
    for ids in (extra, missing):
        vals = key_of(ids)
        assert np.all(np.abs(vals - kth) <= SEL_RTOL * scale), (
            f"{what}: differs beyond ties: {ids[:8]} scores {vals[:8]} vs kth {kth}")
    return extra.size


def check_attn(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    rel = np.max(num / den)
    assert rel <= ATTN_TOL, f"attention max relative error {rel:.3e}"
    return rel
