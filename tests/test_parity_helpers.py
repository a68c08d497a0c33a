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


# Two-spike blocks [a, b, 0, ...]: the rotation gives a + b on even rows and
# a - b on odd rows, so Q*(a - b)/(a + b) is exactly the midpoint between two
# code values on every odd row (E4M3: 432 between 416 and 448; E5M2: 53248
# between 49152 and 57344; INT8: 0.5 between 0 and 1).
TIE_SPIKES = {"e4m3": (55, 1), "e5m2": (27, 1), "int8": (255, 253)}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "int8"])
def test_roundtrip_bound_explains_a_flip(oracle_mod, synth_mod, fmt, monkeypatch):
    """The oracle's own round trip passes with no flagged block; one code
    moved to the other side of its rounding tie passes with one flagged
    block; the same step at a code that is not at a tie, three codes down at
    a tie, or a smooth error of 1e-2 over a block, fail."""
    monkeypatch.setattr(parity, "TOTALS", {})
    B, k = 128, 5
    r = synth_mod.WORKLOADS["laplace_2048x1024"].with_shape(256, 1024, seed=6)
    x = synth_mod.generate(r).reshape(-1).copy()
    a, b = TIE_SPIKES[fmt]
    blk = synth_mod.bits_to_f32(x[k * B:(k + 1) * B])
    p = int(np.round(np.log2(np.max(np.abs(blk)) / a)))
    spikes = np.zeros(B, np.float32)
    spikes[:2] = np.ldexp(np.array([a, b], np.float32), p)
    x[k * B:(k + 1) * B] = (spikes.view(np.uint32) >> 16).astype(np.uint16)   # exact in bf16
    xo = oracle_mod.roundtrip_variant(x, B, "taco", fmt).reshape(-1)
    assert parity.compare_roundtrip(oracle_mod.double_to_bf16(xo), x, B, "taco", fmt,
                                    xo=xo)["flip_blocks"] == 0
    c, al, s = oracle_mod.compress(x, B, fmt=fmt)
    c = c.reshape(-1)
    v, vb = parity.code_arguments(x[k * B:(k + 1) * B], B, "taco", fmt, 1.0, 0.0)
    ties = dict(parity.tie_changes(v, vb, fmt))
    assert sorted(ties) == list(range(1, B, 2))                # every odd row is at a tie
    j = 7
    top = 0                                                    # even row: Q exactly, no tie

    def moved(i, delta):
        cc = c.copy()
        d = oracle_mod.decode(cc[k * B + i:k * B + i + 1], fmt)[0]
        cc[k * B + i] = oracle_mod.encode(np.array([d + delta], np.float32), fmt)[0]
        assert oracle_mod.decode(cc[k * B + i:k * B + i + 1], fmt)[0] == d + delta
        return oracle_mod.double_to_bf16(oracle_mod.reconstruct_f64(cc, al, s, B, fmt=fmt))

    vals = parity.code_values(fmt)
    step = ties[j]
    assert parity.compare_roundtrip(moved(j, step), x, B, "taco", fmt, xo=xo)["flip_blocks"] == 1
    dtop = oracle_mod.decode(c[k * B:k * B + 1], fmt)[0]
    below = vals[np.searchsorted(vals, dtop) - 1]
    with pytest.raises(AssertionError, match="rounding ties"):
        parity.compare_roundtrip(moved(top, below - dtop), x, B, "taco", fmt, xo=xo)
    dj = oracle_mod.decode(c[k * B + j:k * B + j + 1], fmt)[0]
    three = vals[np.searchsorted(vals, dj) - 3]                # three codes down
    with pytest.raises(AssertionError, match="rounding ties"):
        parity.compare_roundtrip(moved(j, three - dj), x, B, "taco", fmt, xo=xo)
    smooth = xo.copy()
    smooth[k * B:(k + 1) * B] *= 1 + 1e-2
    with pytest.raises(AssertionError):
        parity.compare_roundtrip(oracle_mod.double_to_bf16(smooth), x, B, "taco", fmt, xo=xo)


def test_roundtrip_flip_below_the_code_domain_noise(oracle_mod, synth_mod):
    """A tie flip whose change is smaller than the bf16 noise of the block in
    the rotated domain, yet takes an element near zero past its bound
    (block 623 of the GPT-2.7B row-parallel workload at 139 x 9728, seed
    699807680, B = 512): the flip at element 274 alone, and with the tie at
    element 4 flipped too, are explained."""
    r = synth_mod.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(139, 9728, seed=699807680)
    xb = synth_mod.generate(r).reshape(-1)[623 * 512:624 * 512].copy()
    B = 512
    assert xb.size == B
    xo = oracle_mod.roundtrip_variant(xb, B, "taco", "e4m3").reshape(-1)
    c, al, s = oracle_mod.compress(xb, B)
    v, vb = parity.code_arguments(xb, B, "taco", "e4m3", 1.0, 0.0)
    ties = dict(parity.tie_changes(v, vb, "e4m3"))
    assert sorted(ties) == [4, 274]
    for flips in ([274], [4, 274]):
        cc = c.reshape(-1).copy()
        for j in flips:
            d = oracle_mod.decode(cc[j:j + 1], "e4m3")[0]
            cc[j] = oracle_mod.encode(np.array([d + ties[j]], np.float32), "e4m3")[0]
        y = oracle_mod.double_to_bf16(oracle_mod.reconstruct_f64(cc, al, s, B))
        assert parity.compare_roundtrip(y, xb, B, "taco", "e4m3", xo=xo)["flip_blocks"] == 1


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


def test_roundtrip_one_flip_of_a_coarse_variant(oracle_mod, synth_mod):
    """ASH alone in INT8 has codes -3..3 on this gradient tensor (28 x 2560,
    seed 993876353, B = 512): block 23's one rounding tie, flipped, moves the
    whole tensor's relative RMS by more than 1e-3; the flip is explained and
    the RMS is taken with it applied."""
    import math
    r = synth_mod.WORKLOADS["grad_8192x8192"].with_shape(28, 2560, seed=993876353)
    x = synth_mod.generate(r).reshape(-1)
    B, k = 512, 23
    xo = oracle_mod.roundtrip_variant(x, B, "ash", "int8").reshape(-1)
    xb = x[k * B:(k + 1) * B]
    v, vb = parity.code_arguments(xb, B, "ash", "int8", 1.0, 0.0)
    ties = parity.tie_changes(v, vb, "int8")
    assert len(ties) == 1
    j, d = ties[0]
    a, _, _ = oracle_mod.ash_block(xb, B)
    change = np.zeros(B)
    change[j] = d / float(np.float32(a))               # code domain -> x: 1/alpha
    y = xo.copy()
    y[k * B:(k + 1) * B] += oracle_mod.fwht(change) / math.sqrt(B)
    yb = oracle_mod.double_to_bf16(y)
    ref = synth_mod.bits_to_f32(oracle_mod.double_to_bf16(xo)).astype(np.float64)
    assert parity.rel_rms(synth_mod.bits_to_f32(yb).astype(np.float64), ref) > parity.RECON_RTOL
    assert parity.compare_roundtrip(yb, x, B, "ash", "int8", xo=xo)["flip_blocks"] == 1


def test_owner_step_exact_ties(oracle_mod, synth_mod):
    """Two payloads with no own partial (Qwen-7B activation workload, 4 x 512,
    seed 619818529, B = 512): the rotated sum of block 1 sits exactly on a
    midpoint between two E4M3 codes at three elements.  All three flipped
    (more than the per-case bound on 2048 elements allows) pass as exact
    ties; a flip that is at no tie still fails."""
    rows, cols, B, seed = 4, 512, 512, 619818529
    r = synth_mod.WORKLOADS["qwen7b_act_16384x3584"].with_shape(rows, cols, seed=seed)
    pays = [oracle_mod.compress(synth_mod.generate(r.with_shape(rows, cols, seed=seed + 1 + p)), B)
            for p in range(2)]
    c, a, s = parity.oracle_reduce_compress(None, pays, B)
    x = sum(oracle_mod.reconstruct_f64(pc, pa, ps, B).reshape(-1, B)[1] for pc, pa, ps in pays)
    R = oracle_mod.fwht(x)
    v = 448.0 * R / np.max(np.abs(R))
    ties = parity.tie_changes(v, 1e-12 * np.abs(v), "e4m3")   # exact up to the oracle's rounding
    assert len(ties) == 3 and parity.allowed_flips(rows * cols, parity.OWNER_FLIP_RATE) < 3
    bad = c.copy()
    for j, d in ties:
        o = oracle_mod.decode(c[B + j:B + j + 1])[0]
        bad[B + j] = oracle_mod.encode(np.array([o + d], np.float32))[0]
        assert bad[B + j] != c[B + j]
    assert parity.compare_reduce(None, pays, B, bad, a, s)["flips"] == 3
    far = c.copy()
    far[5] ^= 0x02
    with pytest.raises(AssertionError):
        parity.compare_reduce(None, pays, B, far, a, s)
