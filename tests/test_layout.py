"""The indexer-K tile layout's host helpers (fp4_kv_cache_csa2_amd/layout.py): records and
tiles convert both ways, and every byte sits where include/csa2.h places it (entry j in tile
j // 32 at slot e = j % 32: payload bytes 16p .. 16p + 15 at 512p + 16e, scale bytes at
2048 + 4e)."""
import numpy as np
import pytest

from fp4_kv_cache_csa2_amd import layout


@pytest.mark.parametrize("n", [1, 31, 32, 33, 77, 640])
def test_round_trip(n):
    rec = np.random.default_rng(n).integers(0, 256, (n, 68), dtype=np.uint8)
    tiles = layout.records_to_tiles(rec)
    assert tiles.shape == ((n + 31) // 32, 2176)
    assert np.array_equal(layout.tiles_to_records(tiles, n), rec)
    # slots past n are zero
    assert not layout.tiles_to_records(tiles, tiles.shape[0] * 32)[n:].any()


def test_byte_positions():
    n = 100
    rec = np.random.default_rng(7).integers(0, 256, (n, 68), dtype=np.uint8)
    tiles = layout.records_to_tiles(rec)
    for j in range(n):
        t, e = divmod(j, 32)
        for p in range(4):
            assert np.array_equal(tiles[t, 512 * p + 16 * e:512 * p + 16 * e + 16], rec[j, 16 * p:16 * p + 16])
        assert np.array_equal(tiles[t, 2048 + 4 * e:2048 + 4 * e + 4], rec[j, 64:])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        layout.records_to_tiles(np.zeros((4, 64), np.uint8))
    with pytest.raises(ValueError):
        layout.tiles_to_records(np.zeros((1, 2176), np.uint8), 33)
