"""Pins of the oracle's other code formats: E5M2 (the format ablation of the
TACO paper, section 5.3.2; format from section 2.3 / Figure 3) and INT8 (the
fallback of section 6 for hardware without FP8; quantiser of section 2.3 /
Eq. 1), each used in place of E4M3 in the otherwise unchanged Eq. 5-13.

Pinned against: IEEE binary16 (E5M2 is its upper byte) through numpy, torch's
float8_e5m2 decoder and encoder, numpy's round-half-even, an exhaustive
nearest-value search over every binary32 pattern, a hand-worked block
(tests/golden/formats_worked_b4.txt), closed forms and error bounds.
"""
import math

import numpy as np
import pytest

import synth
from conftest import exhaustive_check, read_golden, torch_e5m2_table

FORMATS = ("e4m3", "e5m2", "int8")
QMAX = {"e4m3": 448.0, "e5m2": 57344.0, "int8": 127.0}


def f32_bits_to_bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------- E5M2 -----

def e5m2_from_float16() -> np.ndarray:
    """E5M2 code c has the bit layout of the binary16 pattern c << 8."""
    return (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)


def test_e5m2_decode_is_upper_byte_of_binary16(oracle_mod):
    ours = oracle_mod.decode(np.arange(256, dtype=np.uint8), "e5m2")
    ref = e5m2_from_float16()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[0x7B] == 57344.0 and np.isinf(ours[0x7C]) and np.isinf(ours[0xFC])
    assert np.nanmax(ours[np.isfinite(ours)]) == 57344.0 == oracle_mod.qmax("e5m2")
    assert ours[0x01] == 2.0 ** -16 and ours[0x04] == 2.0 ** -14


def test_e5m2_decode_matches_torch(oracle_mod):
    ours = oracle_mod.decode(np.arange(256, dtype=np.uint8), "e5m2")
    ref = torch_e5m2_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e5m2_encode_inverts_decode_on_every_finite_code(oracle_mod):
    codes = np.array([c for c in range(256) if (c & 0x7F) <= 0x7B], np.uint8)
    vals = oracle_mod.decode(codes, "e5m2").astype(np.float32)
    assert np.array_equal(oracle_mod.encode(vals, "e5m2"), codes)


def test_e5m2_midpoints_round_to_even(oracle_mod):
    vals = oracle_mod.decode(np.arange(0x7C, dtype=np.uint8), "e5m2")
    for c in range(0x7B):
        lo, hi = vals[c], vals[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        got = oracle_mod.encode(np.array([mid, below, above, -mid], np.float32), "e5m2")
        assert got[0] == even and got[1] == c and got[2] == c + 1, (c, got)
        assert got[3] == (even | 0x80)


def test_e5m2_saturation_nan_and_zero(oracle_mod):
    big = np.array([57344.0, 61439.0, 61440.0, 65536.0, 1e30, np.inf], np.float32)
    assert np.all(oracle_mod.encode(big, "e5m2") == 0x7B)
    assert np.all(oracle_mod.encode(-big, "e5m2") == 0xFB)
    assert (oracle_mod.encode(np.array([np.nan], np.float32), "e5m2")[0] & 0x7F) > 0x7C
    tiny = np.array([0.0, -0.0, 2.0 ** -17, -(2.0 ** -17), 1.5 * 2.0 ** -17], np.float32)
    assert list(oracle_mod.encode(tiny, "e5m2")) == [0x00, 0x80, 0x00, 0x80, 0x01]


def test_e5m2_encode_matches_torch_on_random_values(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(99)
    n = 400_000
    mag = np.exp2(rng.uniform(-20, np.log2(61000.0), n))
    v = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(oracle_mod.encode(v, "e5m2"), ref)


def test_e5m2_encode_exhaustive_every_float32(oracle_mod):
    table = e5m2_from_float16()[:0x7C].copy()
    assert np.all(np.diff(table) > 0) and table[-1] == 57344.0
    bad, first = exhaustive_check(oracle_mod.encode_function_address("e5m2"), table,
                                  twos=False, nan_lo=0x7D)
    assert bad == 0, f"{bad} mismatches, first pattern 0x{first:08x}"


def test_e5m2_error_within_half_ulp(oracle_mod):
    """Two mantissa bits: |v - Q(v)| <= 2^(floor(log2|v|) - 3) in the normal range."""
    rng = np.random.default_rng(5)
    v = np.exp2(rng.uniform(-14, np.log2(57000.0), 200_000)).astype(np.float32)
    q = oracle_mod.decode(oracle_mod.encode(v, "e5m2"), "e5m2")
    half_ulp = np.exp2(np.floor(np.log2(v.astype(np.float64))) - 3)
    assert np.all(np.abs(v.astype(np.float64) - q) <= half_ulp)


# --------------------------------------------------------------- INT8 -----

def test_int8_decode_is_twos_complement(oracle_mod):
    ours = oracle_mod.decode(np.arange(256, dtype=np.uint8), "int8")
    ref = np.arange(256, dtype=np.uint8).view(np.int8).astype(np.float64)
    assert np.array_equal(ours, ref)
    assert oracle_mod.qmax("int8") == 127.0


def test_int8_encode_is_round_half_even_clamped(oracle_mod):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-140, 140, 300_000),
                        np.arange(-130, 130) + 0.5,               # exact ties
                        np.arange(-130, 131, dtype=np.float64)]).astype(np.float32)
    want = np.clip(np.rint(v.astype(np.float64)), -127, 127).astype(np.int8).view(np.uint8)
    assert np.array_equal(oracle_mod.encode(v, "int8"), want)
    assert list(oracle_mod.encode(np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5], np.float32),
                                  "int8")) == [0, 2, 2, 0, 0xFE, 0xFE]


def test_int8_encode_exhaustive_every_float32(oracle_mod):
    table = np.arange(128, dtype=np.float64)
    bad, first = exhaustive_check(oracle_mod.encode_function_address("int8"), table,
                                  twos=True, nan_lo=0)
    assert bad == 0, f"{bad} mismatches, first pattern 0x{first:08x}"


# -------------------------------------------------- operator per format ----

def test_worked_block_every_format(oracle_mod):
    """Eq. 5-13 on x = [1, 2, 3, 4], worked by hand for each format."""
    x = f32_bits_to_bf16([1.0, 2.0, 3.0, 4.0])
    rows = read_golden("formats_worked_b4.txt")
    assert [r[0] for r in rows] == list(FORMATS)
    alpha64 = 1.0 / math.sqrt(7.5 + 1e-20)
    for fmt, qm, *rest in rows:
        qm = float(qm)
        codes_want = np.array([int(c, 16) for c in rest[:4]], np.uint8)
        hd = np.array([float(v) for v in rest[4:]])
        assert oracle_mod.qmax(fmt) == qm
        codes, alpha, scale = oracle_mod.compress(x, 4, fmt=fmt)
        assert np.array_equal(codes, codes_want), (fmt, codes)
        assert alpha[0] == np.float32(alpha64)
        assert scale[0] == np.float32(5.0 * alpha64 / qm)
        g = oracle_mod.reconstruct_f64(codes, alpha, scale, 4, fmt=fmt)
        want = hd * 5.0 / (2.0 * qm)
        # alpha and s travel as float32: their ratio carries ~2^-23.
        assert np.allclose(g, want, rtol=2.0 ** -22, atol=0), (fmt, g, want)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("B", [32, 256])
def test_constant_block_reconstructs_exactly(oracle_mod, fmt, B):
    """x = c 1: Z = alpha c sqrt(B) e_0, so the only nonzero code is +-Q_max and
    G' = c (up to the float32 alpha and s)."""
    c = np.float32(-0.375)
    x = f32_bits_to_bf16(np.full(B, c, np.float32))
    codes, alpha, scale = oracle_mod.compress(x, B, fmt=fmt)
    d = oracle_mod.decode(codes, fmt)
    assert d[0] == -QMAX[fmt] and np.all(d[1:] == 0)
    g = oracle_mod.reconstruct_f64(codes, alpha, scale, B, fmt=fmt)
    assert np.allclose(g, c, rtol=2.0 ** -21, atol=0)


@pytest.mark.parametrize("fmt", FORMATS)
def test_dual_scale_uses_the_full_range(oracle_mod, synth_mod, fmt):
    """Eq. 9: every block with a nonzero rotated value has a code of magnitude
    exactly Q_max, and none larger."""
    r = synth.WORKLOADS["grad_8192x8192"].with_shape(8, 4096, seed=31)
    x = synth.generate(r)
    codes, alpha, scale = oracle_mod.compress(x, 256, fmt=fmt)
    d = np.abs(oracle_mod.decode(codes, fmt)).reshape(-1, 256)
    nz = scale > 0
    assert np.all(d.max(axis=1)[nz] == QMAX[fmt])
    assert np.all(d[~nz] == 0)


@pytest.mark.parametrize("fmt,B", [("e5m2", 128), ("int8", 128), ("int8", 512), ("e5m2", 32)])
def test_reconstruction_error_within_quantiser_bound(oracle_mod, synth_mod, fmt, B):
    """The transform is orthonormal, so ||G' - G|| = ||Z-hat - Z|| / alpha, and
    each rotated value is off by at most half a code step times s:
    INT8 steps are 1; E5M2 steps are 2^(e-2) for values in [2^e, 2^(e+1)),
    2^-16 below 2^-14."""
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(4, 3584, seed=41)
    x = synth.generate(r)
    g = synth.bits_to_f32(x).astype(np.float64).reshape(-1, B)
    codes, alpha, scale = oracle_mod.compress(x, B, fmt=fmt)
    gp = oracle_mod.reconstruct_f64(codes, alpha, scale, B, fmt=fmt).reshape(-1, B)
    for k in range(g.shape[0]):
        _, _, z = oracle_mod.ash_block(x.reshape(-1)[k * B:(k + 1) * B], B)
        v = np.abs(z / (float(np.max(np.abs(z))) / QMAX[fmt]))
        if fmt == "int8":
            half = np.full(B, 0.5)
        else:
            e = np.floor(np.log2(np.maximum(v, 2.0 ** -14)))
            half = np.exp2(e - 3)
        bound = float(np.linalg.norm(half * scale[k])) / alpha[k] + 1e-6 * np.linalg.norm(g[k])
        err = float(np.linalg.norm(gp[k] - g[k]))
        assert err <= bound, (k, err, bound)


@pytest.mark.parametrize("fmt", ["e5m2", "int8"])
def test_owner_step_of_one_payload_is_its_recompression(oracle_mod, fmt):
    """Owner step with no own partial and a single payload: X is that
    payload's reconstruction, so the result equals compressing it."""
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(2, 1024, seed=51)
    x = synth.generate(r)
    pay = oracle_mod.compress(x, 128, fmt=fmt)
    g = oracle_mod.reconstruct_f64(*pay, 128, fmt=fmt)
    got = oracle_mod.reduce_compress(None, [pay], 128, fmt=fmt)
    want = oracle_mod.compress_f64(g, 128, fmt=fmt)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_formats_differ_only_in_quantiser(oracle_mod):
    """alpha is the same for every format (Eq. 6-7 do not see the format), and
    s scales with 1 / Q_max."""
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(2, 2560, seed=61)
    x = synth.generate(r)
    out = {f: oracle_mod.compress(x, 128, fmt=f) for f in FORMATS}
    for f in FORMATS[1:]:
        assert np.array_equal(out[f][1], out["e4m3"][1])
        ratio = out[f][2].astype(np.float64) * QMAX[f] / (out["e4m3"][2].astype(np.float64) * 448.0)
        assert np.allclose(ratio, 1.0, rtol=2.0 ** -22)
