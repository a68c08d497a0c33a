"""The comparison helpers of the GPU parity tests, on values whose answers
are fixed by the formats (no GPU needed)."""
import numpy as np
import pytest

import parity


def test_reachable_codes(oracle_mod):
    # E4M3: 1.0625 is the tie between 1.0 (0x38) and 1.125 (0x39).
    assert parity.reachable(0x38, 1.0625, 1e-6) and parity.reachable(0x39, 1.0625, 1e-6)
    assert not parity.reachable(0x3A, 1.0625, 1e-6)
    assert not parity.reachable(0x39, 1.0, 1e-3)
    assert parity.reachable(0x39, 1.0, 0.07)        # the bound reaches past the tie
    # Negative values mirror positive ones.
    assert parity.reachable(0xB8, -1.0625, 1e-6) and not parity.reachable(0x38, -1.0625, 1e-6)
    # E5M2 subnormal range: 0x16, 0x17, 0x18 are 1.5, 1.75 and 2 times 2^-10.
    vals = oracle_mod.decode(np.array([0x16, 0x17, 0x18], np.uint8), "e5m2")
    assert np.array_equal(vals, np.array([1.5, 1.75, 2.0]) * 2.0 ** -10)
    assert parity.reachable(0x18, 1.6e-3, 4e-4, "e5m2")
    assert not parity.reachable(0x18, 1.6e-3, 1e-5, "e5m2")
    # Both zero codes decode to zero: reachable around zero.
    assert parity.reachable(0x80, 1e-12, 1e-11) and parity.reachable(0x00, -1e-12, 1e-11)
    # INT8: q = round(v), ties to even.
    assert parity.reachable(2, 2.5, 1e-9, "int8") and parity.reachable(3, 2.5, 1e-9, "int8")
    assert not parity.reachable(3, 2.4, 1e-3, "int8")


def test_allowed_flips_is_a_poisson_bound():
    assert parity.allowed_flips(0) == 1.0
    assert parity.allowed_flips(100_000) == pytest.approx(1.0 + 3.0 + 1.0)
    n = 20_000_000
    assert parity.allowed_flips(n) == pytest.approx(200 + 3 * np.sqrt(200) + 1)
