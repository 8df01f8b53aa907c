"""Pins for the oracle's storage formats and closed-form accounting (CPU only).

Each test checks the oracle against something other than itself: numbers the pages
print (tests/golden/pages_numbers.txt), torch's own float8 conversions, the MX scale
rule evaluated with numpy's frexp, and invariants of nearest-even rounding."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.txt")


def golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("|")[0].strip()
        if not line or line.startswith("#"):
            continue
        k, v = [s.strip() for s in line.split("=")]
        vals[k] = float(v)
    return vals


G = golden()


def test_entry_sizes_match_pages():
    assert oracle.entry_bytes(512, 16) == G["main_kv_entry_bytes"] == 288
    assert oracle.entry_bytes(128, 32) == G["indexer_k_entry_bytes"] == 68
    assert 512 // 2 == G["main_kv_payload_bytes"] and 512 // 16 == G["main_kv_scale_bytes"]


def test_bytes_per_token_ledger():
    # three m=2 source layers and one m=1 source layer
    ratios = [2, 2, 2, 1]
    assert sum(1.0 / m for m in ratios) == G["sum_inv_ratio_source_layers"]
    main = sum(oracle.entry_bytes(512, 16) / m for m in ratios)
    idx = sum(oracle.entry_bytes(128, 32) / m for m in ratios)
    assert main == G["main_kv_bytes_per_token"]
    assert idx == G["indexer_bytes_per_token"]
    assert main + idx == G["global_kv_bytes_per_token"] == 890
    enc = 3 * (oracle.entry_bytes(512, 16) + oracle.entry_bytes(128, 32)) / 2
    dec = oracle.entry_bytes(512, 16) + oracle.entry_bytes(128, 32)
    assert enc == G["encoder_layers_subtotal"] and dec == G["decoder_layer_subtotal"]
    assert abs(890 * 1e6 / 1e9 - G["resident_gb_at_1m_tokens"]) < 1e-12


def test_v4flash_chain_uses_same_entry_formula():
    v4 = 448 * 1 + 64 * 2 + 8
    assert v4 == G["v4flash_main_entry_bytes"]
    b = 21 * (v4 + oracle.entry_bytes(128, 32)) / 4 + 20 * v4 / 128
    assert b == G["v4flash_bytes_per_token"]
    assert round(b / 890, 2) == G["net_reduction_factor"]


def test_max_representable_magnitude():
    top_scale = oracle.e4m3_value(0x7E)
    top_elem = oracle.e2m1_value(7)
    assert top_scale == G["e4m3_max_scale"] and top_elem == G["e2m1_max_magnitude"]
    assert top_scale * top_elem == G["max_representable_magnitude"] == 2688
    assert np.sqrt(512) == pytest.approx(G["rms_bound_sqrt512"], abs=0.05)


def test_indexer_mac_count_closed_form():
    assert 32 * 128 * 1_000_000 == pytest.approx(G["indexer_mac_per_query_layer_1m"], rel=0.03)
    assert G["candidate_topk_blocks"] * G["candidate_block_size"] == G["candidate_pool_positions"]


def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e8m0_decode_all_codes_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0_value(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])


def _e4m3_probe_values(rng):
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = (grid[1:] + grid[:-1]) / 2
    probe = [grid, mids]
    for v in (mids, grid):
        f = v.astype(np.float32)
        probe += [np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(0))]
    probe.append(rng.uniform(0, 448, 20000))
    probe.append(np.exp2(rng.uniform(-14, 8.8, 20000)))
    x = np.concatenate(probe).astype(np.float32)
    return x[(x >= 0) & (x <= 448)]


def test_e4m3_encode_vs_torch_rne():
    rng = np.random.default_rng(7)
    x = _e4m3_probe_values(rng)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    for v in (448.0, 449.0, 464.0, 500.0, 1e6, float("inf")):
        assert oracle.e4m3_encode(v) == 0x7E


def test_e2m1_codes_roundtrip_and_midpoints():
    grid = [oracle.e2m1_value(c) for c in range(8)]
    assert grid == sorted(grid) and grid[0] == 0.0 and grid[-1] == G["e2m1_max_magnitude"]
    for S in (1.0, 0.375, 2.0 ** -9, 448.0, 2.0 ** -5):
        for c in range(16):
            v = oracle.e2m1_value(c)
            code = oracle.e2m1_encode(np.float32(v * S), S)
            # exact grid points map to themselves (negative zero canonicalises to +0)
            assert code == (0 if (c & 7) == 0 else c)
        # the switch between neighbours sits exactly at the midpoint; ties go to the even code
        for c in range(7):
            mid = np.float32((grid[c] + grid[c + 1]) / 2 * S)
            even = c if c % 2 == 0 else c + 1
            assert oracle.e2m1_encode(mid, S) == even
            assert oracle.e2m1_encode(np.nextafter(mid, np.float32(0)), S) == c
            assert oracle.e2m1_encode(np.nextafter(mid, np.float32(np.inf)), S) == c + 1
        assert oracle.e2m1_encode(np.float32(100 * S), S) == 7
        assert oracle.e2m1_encode(np.float32(-100 * S), S) == 15


def test_e2m1_encode_monotone_and_error_bound():
    rng = np.random.default_rng(3)
    S = 0.3125
    x = np.sort(rng.uniform(0, 6 * S, 4000).astype(np.float32))
    codes = np.array([oracle.e2m1_encode(v, S) for v in x])
    assert np.all(np.diff(codes) >= 0)
    recon = np.array([oracle.e2m1_value(c) for c in codes]) * S
    assert np.max(np.abs(recon - x)) <= 1.0 * S  # the largest half-gap is between 4 and 6
    neg = np.array([oracle.e2m1_encode(-v, S) for v in x])
    assert np.all((neg == codes) | (neg == (codes | 8)))
    assert np.all(neg[codes > 0] == (codes[codes > 0] | 8))


def test_e8m0_scale_rule_vs_frexp():
    rng = np.random.default_rng(5)
    amax = np.concatenate([np.exp2(rng.uniform(-120, 120, 5000)), 2.0 ** np.arange(-120, 121)]).astype(np.float32)
    for a in amax:
        code = oracle.e8m0_scale_code(a)
        _, ex = np.frexp(np.float64(a))
        assert code == (ex - 1) - 2 + 127
        X = oracle.e8m0_value(code)
        assert 4 * X <= a < 8 * X  # MX: the block max lands in the top binade of E2M1
    assert oracle.e8m0_scale_code(0.0) == 0
