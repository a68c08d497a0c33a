"""Pins of the oracle's E4M3 codec (the Cvt_FP8 / Cvt_FP32 of Eq. 10-11 in the
TACO paper, section 4.3; format from section 2.3 / Figure 3 / Eq. 4).

Pinned against: hand-written format values (tests/golden), torch's
float8_e4m3fn decoder and encoder (a library routine), an exhaustive
nearest-value search over every binary32 pattern, and the Eq. 3 error bound.
"""
import ctypes
import math

import numpy as np
import pytest

from conftest import exhaustive_check, read_golden, torch_e4m3_table


def test_decode_known_values(oracle_mod):
    for code_s, val_s in read_golden("e4m3_values.txt"):
        code = int(code_s, 16)
        got = oracle_mod.e4m3_decode(np.array([code], np.uint8))[0]
        if val_s == "nan":
            assert math.isnan(got), hex(code)
        else:
            want = float(val_s)
            assert got == want, (hex(code), got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), hex(code)


def test_decode_matches_torch_all_codes(oracle_mod):
    ours = oracle_mod.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = torch_e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[0x7E] == 448.0 and np.nanmax(ours) == 448.0


def test_encode_inverts_decode_on_every_finite_code(oracle_mod):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle_mod.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle_mod.e4m3_encode(vals), codes)


def test_midpoints_round_to_even_and_neighbours_to_nearest(oracle_mod):
    vals = oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8))
    for c in range(126):
        lo, hi = vals[c], vals[c + 1]
        mid = np.float32((lo + hi) / 2)           # exact: 5 significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        got = oracle_mod.e4m3_encode(np.array([mid, below, above, -mid], np.float32))
        assert got[0] == even, (c, lo, hi)
        assert got[1] == c and got[2] == c + 1, (c, got)
        assert got[3] == (even | 0x80)


def test_saturation_and_nan(oracle_mod):
    big = np.array([448.0, 448.5, 463.9, 464.0, 479.0, 480.0, 1e30,
                    np.finfo(np.float32).max, np.inf], np.float32)
    assert np.all(oracle_mod.e4m3_encode(big) == 0x7E)
    assert np.all(oracle_mod.e4m3_encode(-big) == 0xFE)
    assert oracle_mod.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F
    # Signed zero and tiny values keep their sign; values at or below 2^-10
    # (half the smallest subnormal, a tie with 0) round to zero.
    tiny = np.array([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -11,
                     np.nextafter(np.float32(2 ** -10), np.float32(1))], np.float32)
    assert list(oracle_mod.e4m3_encode(tiny)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x01]


def test_encode_matches_torch_on_random_values(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1234)
    n = 400_000
    mag = np.exp2(rng.uniform(-14, np.log2(463.0), n))     # log-uniform magnitudes
    v = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    v = np.concatenate([v, rng.uniform(-463, 463, n).astype(np.float32)])
    ours = oracle_mod.e4m3_encode(v)
    # torch's conversion does not saturate (it gives NaN from 464 on), so the
    # sample stays below 464.
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_exhaustive_every_float32(oracle_mod):
    """All 2^31 non-negative binary32 patterns (and their negatives)."""
    table = torch_e4m3_table()[:127].astype(np.float64).copy()   # library decoder
    assert np.all(np.diff(table) > 0) and table[126] == 448.0
    bad, first = exhaustive_check(oracle_mod.encode_function_address("e4m3"), table,
                                  twos=False, nan_lo=0x7F)
    assert bad == 0, f"{bad} mismatches, first pattern 0x{first:08x}"


def test_quantisation_error_within_eq3_bound(oracle_mod):
    """Eq. 3: |x - Q(x)| <= ULP(x) = 2^(floor(log2|x|) - m), m = 3 (nearest
    rounding gives half of that) in the normal range."""
    rng = np.random.default_rng(7)
    v = np.exp2(rng.uniform(-6, np.log2(447.0), 200_000)).astype(np.float32)
    q = oracle_mod.e4m3_decode(oracle_mod.e4m3_encode(v))
    ulp = np.exp2(np.floor(np.log2(v.astype(np.float64))) - 3)
    err = np.abs(v.astype(np.float64) - q)
    assert np.all(err <= ulp)
    assert np.all(err <= 0.5 * ulp)
