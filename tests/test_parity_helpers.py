"""The comparison helpers of the GPU parity tests, on values whose answers
are fixed by the formats (no GPU needed)."""
import numpy as np
import pytest

import parity


@pytest.fixture(autouse=True)
def own_totals(monkeypatch):
    """These tests plant mismatches: keep them out of the session's totals."""
    monkeypatch.setattr(parity, "TOTALS", {})


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


def test_session_totals_by_kind_and_format(monkeypatch):
    monkeypatch.setattr(parity, "TOTALS", {})
    parity.tally("compress", "e4m3", 3, 1_000_000)
    parity.tally("compress", "e4m3", 2, 1_000_000)
    parity.tally("owner", "e4m3", 15, 2_000_000)
    lines, ok = parity.session_check()
    assert ok and len(lines) == 2
    assert "[compress e4m3]: 5 in 2000000" in lines[0]
    parity.tally("compress", "int8", 11, 1_000_000)       # 1.1e-5 > 1e-5
    lines, ok = parity.session_check()
    assert not ok and any("EXCEEDED" in ln for ln in lines)


def test_every_differing_code_is_verified(monkeypatch, oracle_mod, synth_mod):
    """compare_compress checks each differing code, however many there are."""
    r = synth_mod.WORKLOADS["laplace_2048x1024"].with_shape(64, 1024, seed=3)
    x = synth_mod.generate(r)
    c, a, s = oracle_mod.compress(x, 128)
    bad = c.reshape(-1).copy()
    idx = np.arange(0, bad.size, 250)[:260]
    bad[idx] ^= 1                                    # 260 planted changes
    seen = []
    monkeypatch.setattr(parity, "allowed_flips", lambda n, rate=1e-5: 1e9)
    monkeypatch.setattr(parity, "_tie_ok", lambda xb, cg, co, j, B, fmt="e4m3":
                        (seen.append(j) or True, ""))
    monkeypatch.setattr(parity, "TOTALS", {})
    st = parity.compare_compress(x, 128, bad, a, s)
    assert st["flips"] == 260 and len(seen) == 260
    # Unpatched, the first planted change that is not at a tie fails.
    monkeypatch.undo()
    monkeypatch.setattr(parity, "TOTALS", {})
    with pytest.raises(AssertionError):
        parity.compare_compress(x, 128, bad, a, s)


def test_threaded_oracle_equals_one_call(oracle_mod, synth_mod):
    r = synth_mod.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(300, seed=4)
    x = synth_mod.generate(r)
    assert len(parity.block_runs(x.size // 128)) > 1
    c1, a1, s1 = oracle_mod.compress(x, 128)
    c2, a2, s2 = parity.oracle_compress(x, 128)
    assert np.array_equal(c1.reshape(-1), c2) and np.array_equal(a1, a2)
    assert np.array_equal(s1, s2)


def test_accumulate_bound(oracle_mod, synth_mod):
    """The oracle's own accumulator passes; an element moved by a few float32
    units passes; one moved by 1e-4 of its value fails."""
    r = synth_mod.WORKLOADS["gpt175b_hidden_32768x12288"].with_shape(4, 3072)
    pays = [oracle_mod.compress(synth_mod.generate(r, seed=40 + p), 256) for p in range(3)]
    acc0 = (np.random.default_rng(5).standard_normal(4 * 3072) * 0.01).astype(np.float32)
    ref = acc0.copy()
    for c, a, s in pays:
        oracle_mod.decompress_accumulate(c, a, s, 256, ref)
    parity.compare_accumulate(ref, acc0, pays, 256)
    near = ref.copy()
    near[17] = np.nextafter(np.nextafter(near[17], np.float32(np.inf)), np.float32(np.inf))
    parity.compare_accumulate(near, acc0, pays, 256)
    far = ref.copy()
    far[1000] *= np.float32(1 + 1e-4)
    with pytest.raises(AssertionError):
        parity.compare_accumulate(far, acc0, pays, 256)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "int8"])
def test_roundtrip_bound_explains_a_flip(oracle_mod, synth_mod, fmt, monkeypatch):
    """The oracle's own round trip passes with no flagged block; a round trip
    whose codes differ from the oracle's by one adjacent code in one block
    passes with one flagged block; three code steps, or a smooth error of
    1e-2 over a block, fail."""
    monkeypatch.setattr(parity, "TOTALS", {})
    B = 128
    # (large enough that one changed top code stays within the RMS tolerance)
    r = synth_mod.WORKLOADS["laplace_2048x1024"].with_shape(256, 1024, seed=6)
    x = synth_mod.generate(r)
    xo = oracle_mod.roundtrip_variant(x, B, "taco", fmt).reshape(-1)
    y = oracle_mod.double_to_bf16(xo)
    assert parity.compare_roundtrip(y, x, B, "taco", fmt, xo=xo)["flip_blocks"] == 0
    c, a, s = oracle_mod.compress(x, B, fmt=fmt)
    c = c.reshape(-1).copy()
    k = 5
    # The block's largest code (+-Q_max): one step toward zero is visible in
    # every element.
    i = k * B + int(np.argmax(np.abs(oracle_mod.decode(c[k * B:(k + 1) * B], fmt))))
    d = oracle_mod.decode(c[i:i + 1], fmt)[0]
    assert abs(d) == parity.QMAX_OF[fmt]

    def toward_zero(steps):
        cc = c.copy()
        if fmt == "int8" and d < 0:
            cc[i] = (int(c[i]) + steps) & 0xFF
        else:
            cc[i] = int(c[i]) - steps
        return oracle_mod.double_to_bf16(oracle_mod.reconstruct_f64(cc, a, s, B, fmt=fmt))

    assert parity.compare_roundtrip(toward_zero(1), x, B, "taco", fmt, xo=xo)["flip_blocks"] == 1
    with pytest.raises(AssertionError):
        parity.compare_roundtrip(toward_zero(3), x, B, "taco", fmt, xo=xo)
    smooth = xo.copy()
    smooth[k * B:(k + 1) * B] *= 1 + 1e-2
    with pytest.raises(AssertionError):
        parity.compare_roundtrip(oracle_mod.double_to_bf16(smooth), x, B, "taco", fmt, xo=xo)


@pytest.mark.parametrize("variant", ["ds", "tensor", "ash", "hadamard"])
def test_roundtrip_bound_other_variants(oracle_mod, synth_mod, variant):
    """Every variant's own oracle round trip passes with no flagged block."""
    r = synth_mod.WORKLOADS["grad_8192x8192"].with_shape(4, 8192, seed=7)
    x = synth_mod.generate(r)
    for fmt in ("e4m3", "int8"):
        xo = oracle_mod.roundtrip_variant(x, 256, variant, fmt).reshape(-1)
        st = parity.compare_roundtrip(oracle_mod.double_to_bf16(xo), x, 256, variant, fmt, xo=xo)
        assert st["flip_blocks"] == 0


def test_owner_step_helpers(oracle_mod, synth_mod):
    """The threaded oracle owner step equals one call; the oracle's own result
    passes compare_reduce; a code moved away from a tie fails it."""
    r = synth_mod.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(200, seed=8)
    own = synth_mod.generate(r)
    pays = [oracle_mod.compress(synth_mod.generate(r, seed=80 + p), 128) for p in range(2)]
    c1, a1, s1 = oracle_mod.reduce_compress(own, pays, 128)
    c2, a2, s2 = parity.oracle_reduce_compress(own, pays, 128)
    assert np.array_equal(c1.reshape(-1), c2) and np.array_equal(a1, a2) and np.array_equal(s1, s2)
    assert parity.compare_reduce(own, pays, 128, c2, a2, s2)["flips"] == 0
    bad = c2.copy()
    bad[5000] ^= 0x02                          # two codes away: no tie explains it
    with pytest.raises(AssertionError):
        parity.compare_reduce(own, pays, 128, bad, a2, s2)
    assert parity.compare_reduce(None, pays, 128, *parity.oracle_reduce_compress(None, pays, 128))[
        "flips"] == 0


def test_accumulate_n_bound(oracle_mod, synth_mod):
    r = synth_mod.WORKLOADS["gpt175b_hidden_32768x12288"].with_shape(4, 3072)
    pays = [oracle_mod.compress(synth_mod.generate(r, seed=50 + p), 256) for p in range(4)]
    acc0 = (np.random.default_rng(6).standard_normal(4 * 3072) * 0.01).astype(np.float32)
    ref = oracle_mod.decompress_accumulate_n(pays, 256, acc0.copy())
    st = parity.compare_accumulate_n(ref, acc0, pays, 256)
    assert st["max_err_over_block_magnitude"] == 0.0
    far = ref.copy()
    far[333] += np.float32(1e-3 * np.max(np.abs(ref[256:512])))
    with pytest.raises(AssertionError):
        parity.compare_accumulate_n(far, acc0, pays, 256)
