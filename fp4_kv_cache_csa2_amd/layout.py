"""Host-side conversion between 68-byte indexer-K records and the cache's tile layout.

The kernels keep the indexer-K cache (and HISA's block-mean cache) in tiles of 32 entries,
2176 bytes each: plane p (p = 0 .. 3) of a tile holds payload bytes 16p .. 16p + 15 of its 32
entries, 16 bytes per entry, and the last 128 bytes hold the entries' 4-byte E8M0 scale
words (include/csa2.h).  A record is the entry's 64 payload bytes in channel order followed
by its 4 scale bytes.  These helpers only move bytes: they are for building a cache from
records made elsewhere and for reading one back as records.
"""
from __future__ import annotations

import numpy as np

TILE_ENTRIES = 32
TILE_BYTES = 2176
RECORD_BYTES = 68


def records_to_tiles(rec: np.ndarray) -> np.ndarray:
    """uint8 [n, 68] records -> uint8 [ceil(n / 32), 2176] tiles (entries past n zero)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    if rec.ndim != 2 or rec.shape[1] != RECORD_BYTES:
        raise ValueError(f"records must be [n, {RECORD_BYTES}] uint8, got {rec.shape}")
    n = rec.shape[0]
    n_tiles = (n + TILE_ENTRIES - 1) // TILE_ENTRIES
    full = np.zeros((n_tiles * TILE_ENTRIES, RECORD_BYTES), np.uint8)
    full[:n] = rec
    full = full.reshape(n_tiles, TILE_ENTRIES, RECORD_BYTES)
    planes = full[:, :, :64].reshape(n_tiles, TILE_ENTRIES, 4, 16).transpose(0, 2, 1, 3)
    out = np.empty((n_tiles, TILE_BYTES), np.uint8)
    out[:, :2048] = planes.reshape(n_tiles, 2048)
    out[:, 2048:] = full[:, :, 64:].reshape(n_tiles, 128)
    return out


def tiles_to_records(tiles: np.ndarray, n: int) -> np.ndarray:
    """uint8 [n_tiles, 2176] tiles -> the first n entries as uint8 [n, 68] records."""
    tiles = np.ascontiguousarray(tiles, dtype=np.uint8)
    if tiles.ndim != 2 or tiles.shape[1] != TILE_BYTES or tiles.shape[0] * TILE_ENTRIES < n:
        raise ValueError(f"tiles must be [>= {(n + TILE_ENTRIES - 1) // TILE_ENTRIES}, {TILE_BYTES}] uint8, "
                         f"got {tiles.shape}")
    n_tiles = tiles.shape[0]
    rec = np.empty((n_tiles, TILE_ENTRIES, RECORD_BYTES), np.uint8)
    rec[:, :, :64] = tiles[:, :2048].reshape(n_tiles, 4, TILE_ENTRIES, 16).transpose(0, 2, 1, 3).reshape(
        n_tiles, TILE_ENTRIES, 64)
    rec[:, :, 64:] = tiles[:, 2048:].reshape(n_tiles, TILE_ENTRIES, 4)
    return rec.reshape(-1, RECORD_BYTES)[:n]
