"""Pins of the oracle's ablation variants (the round trips the TACO paper
compares its operator with: direct FP8 quantization, section 4.2.1 and the
NVFP8 arm of section 5.2.2; DS and ASH in isolation, section 5.2.2; the
standard Hadamard transform, sections 4.2.1 and 5.3.1; one scale per tensor,
the quantiser of section 2.3 / Eq. 1) and of the fidelity metrics RelL2, Cos,
MaxErr and MSE as the GIFT page ("GIFT: Geometry-Informed Low-precision
Gradient Communication for LLM Pretraining") defines them in Eq. 21.

Pinned against: hand-worked metric values, closed forms of each variant on
blocks whose round trip can be written out, the zero-collapse case the pages
describe, and per-element quantiser bounds.
"""
import math

import numpy as np
import pytest

import synth

QMAX = {"e4m3": 448.0, "e5m2": 57344.0, "int8": 127.0}
FORMATS = ("e4m3", "e5m2", "int8")


def bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# ------------------------------------------------------------ metrics ----

def test_metrics_worked_example(oracle_mod):
    """x = [1, 2, 3, 4], x' = [1, 2, 3, 5]: |x' - x| = 1, |x|^2 = 30,
    |x'|^2 = 39, <x', x> = 34."""
    m = oracle_mod.fidelity([1, 2, 3, 4], [1, 2, 3, 5])
    assert m["rel_l2"] == pytest.approx(1 / math.sqrt(30), rel=1e-15)
    assert m["cos"] == pytest.approx(34 / math.sqrt(30 * 39), rel=1e-15)
    assert m["max_err"] == 1.0
    assert m["mse"] == 0.25


def test_metrics_scaled_copy_and_sign_flip(oracle_mod):
    x = np.array([0.5, -1.0, 2.0, 0.0, 3.0])
    m = oracle_mod.fidelity(x, 2 * x)          # direction kept, error = x
    assert m["rel_l2"] == pytest.approx(1.0, rel=1e-15)
    assert m["cos"] == pytest.approx(1.0, rel=1e-15)
    assert m["max_err"] == 3.0 and m["mse"] == pytest.approx(np.mean(x * x), rel=1e-15)
    m = oracle_mod.fidelity(x, -x)             # opposite direction, error = 2x
    assert m["cos"] == pytest.approx(-1.0, rel=1e-15)
    assert m["rel_l2"] == pytest.approx(2.0, rel=1e-15)
    m = oracle_mod.fidelity(x, x)
    assert m["rel_l2"] == 0.0 and m["max_err"] == 0.0 and m["mse"] == 0.0


# ----------------------------------------------------------- variants ----

@pytest.mark.parametrize("fmt", FORMATS)
def test_taco_variant_is_compress_then_reconstruct(oracle_mod, fmt):
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(2, 2560, seed=71)
    x = synth.generate(r)
    want = oracle_mod.reconstruct_f64(*oracle_mod.compress(x, 128, fmt=fmt), 128, fmt=fmt)
    assert np.array_equal(oracle_mod.roundtrip_variant(x, 128, "taco", fmt), want)


@pytest.mark.parametrize("fmt", FORMATS)
def test_direct_cast_keeps_code_values_and_collapses_tiny_ones(oracle_mod, fmt):
    """Direct quantization: values that are codes come back exactly; values
    below half the smallest nonzero code collapse to zero (RelL2 = 1)."""
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle_mod.decode(codes, fmt)
    ok = np.isfinite(vals) & (np.abs(vals) < 256)        # exact in bf16 below 2^8
    v = np.resize(vals[ok], 128)
    x = bf16(v)
    assert np.array_equal(oracle_mod.roundtrip_variant(x, 128, "direct", fmt), v)
    smallest = np.min(np.abs(vals[np.isfinite(vals) & (vals != 0)]))
    tiny = np.full(128, smallest / 4)
    tiny[::2] *= -1
    y = oracle_mod.roundtrip_variant(bf16(tiny), 128, "direct", fmt)
    assert np.all(y == 0)
    assert oracle_mod.fidelity(tiny, y)["rel_l2"] == 1.0


@pytest.mark.parametrize("fmt", FORMATS)
def test_dual_scale_only_on_code_ratios(oracle_mod, fmt):
    """DS alone: a block whose values are max * (code / Q_max) comes back up
    to the float32 scale: x / s lands on a code (max * 2^-k for the FP8
    formats, max * k / 127 for INT8)."""
    if fmt == "int8":            # max = 127 2^-5, values k 2^-5: exact in bf16
        v = (np.arange(32) * 4 - 1) * 2.0 ** -5
        v[-1] = 127 * 2.0 ** -5
    else:
        v = 3.0 * 2.0 ** -(np.arange(32) % 6)
    v[1::2] *= -1
    m = float(np.max(np.abs(v)))
    x = bf16(v)
    y = oracle_mod.roundtrip_variant(x, 32, "ds", fmt)
    s32 = np.float32(m / QMAX[fmt])
    want = oracle_mod.decode(oracle_mod.encode(np.float32(v / (m / QMAX[fmt])), fmt), fmt) * s32
    assert np.array_equal(y, want)
    assert np.allclose(y, v, rtol=2.0 ** -22)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("B", [32, 128])
def test_ash_alone_on_a_constant_block(oracle_mod, fmt, B):
    """x = c 1: Z = alpha c sqrt(B) e_0 = tau sqrt(B) sign(c) e_0 (eps aside),
    so x' = decode(Cvt(sqrt(B))) / (sqrt(B) alpha) in every element."""
    c = -0.75
    x = bf16(np.full(B, c))
    y = oracle_mod.roundtrip_variant(x, B, "ash", fmt)
    alpha = np.float32(1.0 / math.sqrt(c * c + 1e-20))
    q = oracle_mod.decode(oracle_mod.encode(np.float32([-math.sqrt(B)]), fmt), fmt)[0]
    want = q / math.sqrt(B) / float(alpha)
    assert np.allclose(y, want, rtol=1e-14)


@pytest.mark.parametrize("fmt", FORMATS)
def test_standard_hadamard_on_a_walsh_row(oracle_mod, fmt):
    """x = c h_r (row r of H): H x / sqrt(B) = c sqrt(B) e_r, so
    x' = decode(Cvt(c sqrt(B))) h_r / sqrt(B)."""
    B, r, c = 64, 37, 2.5
    h = sylvester(B)[r]
    y = oracle_mod.roundtrip_variant(bf16(c * h), B, "hadamard", fmt)
    q = oracle_mod.decode(oracle_mod.encode(np.float32([c * math.sqrt(B)]), fmt), fmt)[0]
    assert np.allclose(y, q * h / math.sqrt(B), rtol=1e-14)


def test_standard_hadamard_keeps_low_energy_blocks_low(oracle_mod):
    """The pages' point about the standard rotation: it preserves the L2
    norm, so a low-energy block stays in the low range; with INT8 codes and
    no scale every rotated value rounds to zero (RelL2 = 1)."""
    rng = np.random.default_rng(3)
    v = rng.laplace(0, 0.01, 256)
    x = bf16(v)
    g = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = oracle_mod.roundtrip_variant(x, 256, "hadamard", "int8")
    assert np.all(y == 0) and oracle_mod.fidelity(g, y)["rel_l2"] == 1.0
    # The rotation is an isometry: the rotated block's norm equals the input's.
    z = oracle_mod.fwht(g) / 16.0
    assert np.linalg.norm(z) == pytest.approx(np.linalg.norm(g), rel=1e-14)


def test_tensor_scale_int8_on_exact_multiples(oracle_mod):
    """One scale per tensor with INT8 codes (section 2.3 / Eq. 1): x = k 2^-7,
    k in [-127, 127], max|x| = 127 2^-7, so Delta = 2^-7 and x' = x."""
    k = np.arange(-127, 129)
    k[-1] = 0
    v = k * 2.0 ** -7
    y = oracle_mod.roundtrip_variant(bf16(v), 128, "tensor", "int8")
    assert np.array_equal(y, v)


def test_tensor_scale_uses_the_whole_tensor(oracle_mod):
    """The scale is shared: a block of small values next to one large value
    quantises with the large value's step (error up to Delta / 2)."""
    v = np.concatenate([np.full(32, 0.3), np.zeros(31), [127.0]])
    y = oracle_mod.roundtrip_variant(bf16(v), 32, "tensor", "int8")
    assert y[-1] == 127.0
    assert np.all(y[:32] == 0.0)                      # 0.3 < Delta / 2 = 0.5
    y_ds = oracle_mod.roundtrip_variant(bf16(v), 32, "ds", "int8")
    x03 = float((bf16([0.3]).astype(np.uint32) << 16).view(np.float32)[0])
    assert np.allclose(y_ds[:32], x03, rtol=2.0 ** -22)          # its own block scale


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
def test_ds_error_within_half_a_step(oracle_mod, fmt):
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(2, 3584, seed=72)
    x = synth.generate(r)
    g = synth.bits_to_f32(x).astype(np.float64).reshape(-1, 128)
    y = oracle_mod.roundtrip_variant(x, 128, "ds", fmt).reshape(-1, 128)
    s = np.max(np.abs(g), axis=1, keepdims=True) / QMAX[fmt]
    u = np.abs(g) / s
    if fmt == "int8":
        half = np.full_like(u, 0.5)
    else:
        half = np.exp2(np.floor(np.log2(np.maximum(u, 2.0 ** -6))) - 4)
    # plus |code| times the float32 rounding of s (at most Q_max 2^-24 s)
    assert np.all(np.abs(y - g) <= (half + QMAX[fmt] * 2.0 ** -23) * s)
