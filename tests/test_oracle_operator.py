"""Pins of the oracle's compress / decompress / accumulate (TACO paper,
section 4.2.2 Eq. 5-8, section 4.3 Eq. 9-13, Algorithm 1).

Each property below is something the equations fix independently of how the
oracle evaluates them: the target energy of the rescaled block, energy
preservation of the rotation, exact invertibility without quantisation,
invariances, closed-form results for special blocks, and the per-element
quantisation error bound of Eq. 3 carried through the orthogonal inverse.
"""
import math

import numpy as np
import pytest

EPS = 1e-20
QMAX = 448.0


def f32_to_bits(v):
    import synth
    return synth.f32_to_bits(np.asarray(v, np.float32))


def bits_to_f64(bits):
    import synth
    return synth.bits_to_f32(bits).astype(np.float64)


def laplace_block(rng, B, scale=0.02):
    return f32_to_bits(rng.laplace(0.0, scale, B))


# ------------------------------------------------------ Eq. 6-8 ----------

@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
def test_rescaled_block_energy_hits_target(oracle_mod, B):
    """Eq. 6-7: mean(Gt^2) = tau^2 * m / (m + eps), m = mean(G^2)."""
    rng = np.random.default_rng(B)
    for tau, eps, scale in [(1.0, EPS, 0.02), (3.5, EPS, 1e-4), (1.0, 1e-6, 1e-3), (0.25, 0.0, 5.0)]:
        x = laplace_block(rng, B, scale)
        alpha, gt, z = oracle_mod.ash_block(x, B, tau, eps)
        g = bits_to_f64(x)
        m = np.mean(g ** 2)
        np.testing.assert_allclose(np.mean(gt ** 2), tau ** 2 * m / (m + eps), rtol=1e-13)
        np.testing.assert_allclose(gt, alpha * g, rtol=1e-15)
        # Eq. 8 is orthonormal: the rotation preserves the energy.
        np.testing.assert_allclose(np.sum(z ** 2), np.sum(gt ** 2), rtol=1e-13)


@pytest.mark.parametrize("B", [32, 128, 256, 512])
def test_roundtrip_without_quantisation_is_identity(oracle_mod, B):
    """Eq. 11-13 undo Eq. 7-8 exactly when Z-hat = Z."""
    rng = np.random.default_rng(100 + B)
    for scale in [1e-4, 0.02, 30.0]:
        x = laplace_block(rng, B, scale)
        got = oracle_mod.roundtrip_noquant(x, B, 1.0, EPS)
        np.testing.assert_allclose(got, bits_to_f64(x), rtol=1e-12, atol=1e-300)


# ------------------------------------------------ invariances ------------

@pytest.mark.parametrize("B", [64, 256])
def test_codes_invariant_under_power_of_two_scaling(oracle_mod, B):
    """With eps = 0, x -> 2^k x gives alpha -> 2^-k alpha exactly and leaves
    the rescaled block, hence Z, s and the codes, bit-identical."""
    rng = np.random.default_rng(5)
    x = laplace_block(rng, 8 * B).reshape(8, B)
    c0, a0, s0 = oracle_mod.compress(x, B, 1.0, 0.0)
    for k in [-20, -3, 1, 7, 30]:
        xk = f32_to_bits(bits_to_f64(x) * 2.0 ** k)
        assert np.array_equal(bits_to_f64(xk), bits_to_f64(x) * 2.0 ** k)
        ck, ak, sk = oracle_mod.compress(xk, B, 1.0, 0.0)
        assert np.array_equal(ck, c0)
        assert np.array_equal(sk, s0)
        assert np.array_equal(ak.astype(np.float64), a0.astype(np.float64) * 2.0 ** -k)


@pytest.mark.parametrize("B", [128, 256])
def test_codes_do_not_depend_on_tau(oracle_mod, B):
    """Z/s = Q * Z / max|Z| is free of the common factor alpha (Eq. 7-10), so
    the codes match for any target energy, and alpha, s scale with tau."""
    import synth
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(64)
    x = synth.generate(r)
    c1, a1, s1 = oracle_mod.compress(x, B, 1.0)
    for tau in [0.01, 37.5, 1e6]:
        ct, at, st = oracle_mod.compress(x, B, tau)
        flips = np.count_nonzero(ct != c1)
        # The double-precision Z/s carries rounding noise of ~1e-16 relative;
        # it can only move a code when Z/s sits within that of a tie.
        assert flips <= 2, flips
        np.testing.assert_allclose(at, a1 * tau, rtol=2e-7)
        np.testing.assert_allclose(st, s1 * tau, rtol=2e-7)


# ------------------------------------------------- special blocks --------

@pytest.mark.parametrize("B", [32, 128, 256, 512])
def test_constant_block(oracle_mod, B):
    """H c 1 = (B c, 0, ..., 0): one code at +-Q_max, exact reconstruction."""
    for c in [0.015625, -3.0, 1e-30, 7.5e20]:
        x = f32_to_bits(np.full(B, c))
        cb = float(bits_to_f64(x[:1])[0])          # the bf16 value of c
        codes, alpha, s = oracle_mod.compress(x, B)
        want = np.zeros(B, np.uint8)
        want[0] = 0x7E if c > 0 else 0xFE
        assert np.array_equal(codes, want)
        np.testing.assert_allclose(alpha[0], 1.0 / math.sqrt(cb * cb + EPS), rtol=1e-7)
        np.testing.assert_allclose(s[0], alpha[0] * abs(cb) * math.sqrt(B) / QMAX, rtol=1e-6)
        assert np.array_equal(oracle_mod.decompress(codes, alpha, s, B), x)


@pytest.mark.parametrize("B", [32, 256])
def test_single_spike(oracle_mod, B):
    """x = a e_p gives Z_j = a alpha H[j, p] / sqrt(B): all codes +-Q_max with
    the signs of column p of H, and an exact reconstruction."""
    from scipy.linalg import hadamard
    H = hadamard(B)
    for p, a in [(0, 0.5), (B - 1, -2.0), (B // 3, 1e-3)]:
        xv = np.zeros(B)
        xv[p] = a
        x = f32_to_bits(xv)
        codes, alpha, s = oracle_mod.compress(x, B)
        signs = np.sign(a) * H[:, p]
        assert np.array_equal(codes, np.where(signs > 0, 0x7E, 0xFE).astype(np.uint8))
        assert np.array_equal(oracle_mod.decompress(codes, alpha, s, B), x)


@pytest.mark.parametrize("B", [64, 512])
def test_walsh_row_has_a_single_code(oracle_mod, B):
    """x = a H[r, :] gives Z = a alpha sqrt(B) e_r."""
    from scipy.linalg import hadamard
    H = hadamard(B).astype(np.float64)
    for r, a in [(1, 0.25), (B - 2, -0.75)]:
        x = f32_to_bits(a * H[r])
        codes, alpha, s = oracle_mod.compress(x, B)
        want = np.zeros(B, np.uint8)
        want[r] = 0x7E if a > 0 else 0xFE
        assert np.array_equal(codes, want)
        assert np.array_equal(oracle_mod.decompress(codes, alpha, s, B), x)


def test_zero_block(oracle_mod):
    """All-zero block: alpha = tau / sqrt(eps), s = 0, zero codes, zero output."""
    B = 128
    x = np.zeros(2 * B, np.uint16)
    x[B:] = 0x8000                               # negative zeros too
    codes, alpha, s = oracle_mod.compress(x, B, 2.0)
    assert np.all(codes == 0) and np.all(s == 0)
    np.testing.assert_allclose(alpha, 2.0 / math.sqrt(EPS), rtol=1e-7)
    y = oracle_mod.decompress(codes, alpha, s, B)
    assert np.all(bits_to_f64(y) == 0.0)


def test_exact_zero_rotated_values_encode_as_positive_zero(oracle_mod):
    """Z_j == 0 of either sign encodes as 0x00.  Pairs (-0, +0) followed by a
    constant half make the butterflies produce a negative zero at index 17
    ((-0) - (+0) = -0), next to positive zeros elsewhere."""
    B = 32
    xv = np.zeros(B, np.float32)
    xv[0:16:2] = -0.0
    xv[16:] = 0.75
    _, _, z = oracle_mod.ash_block(f32_to_bits(xv), B)
    assert z[17] == 0 and np.signbit(z[17])      # the case is really exercised
    assert np.any((z == 0) & ~np.signbit(z))
    codes, _, _ = oracle_mod.compress(f32_to_bits(xv), B)
    assert np.all(codes[z == 0] == 0x00)
    # The constant half contributes +-0.75 * 16 at indices 0 and 16 only.
    assert codes[0] == 0x7E and codes[16] == 0xFE and np.count_nonzero(codes) == 2


def test_subnormal_inputs(oracle_mod):
    """bf16 subnormals are exact in double; the block still round-trips within
    the quantisation bound and nothing overflows."""
    B = 128
    rng = np.random.default_rng(9)
    bits = rng.integers(1, 0x7F, B).astype(np.uint16)          # subnormal magnitudes
    bits |= (rng.integers(0, 2, B).astype(np.uint16) << 15)
    codes, alpha, s = oracle_mod.compress(bits, B)
    assert np.isfinite(alpha).all() and (s > 0).all()
    g = oracle_mod.reconstruct_f64(codes, alpha, s, B)
    x = bits_to_f64(bits)
    assert np.linalg.norm(g - x) <= 0.07 * np.linalg.norm(x)


# ------------------------------------------- quantisation error ----------

@pytest.mark.parametrize("B", [128, 256])
def test_error_bound_through_orthogonal_inverse(oracle_mod, B):
    """Per element, |decode(q) - Z/s| <= half an E4M3 spacing (Eq. 3 with
    nearest rounding) plus the float32 rounding of Z/s; and by orthogonality
    of Eq. 8 / Eq. 12, ||G' - G|| = ||Z-hat / alpha32 - Z / alpha||."""
    import synth
    rng_blocks = 96
    x = synth.generate(synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(rng_blocks * B // 2560 + 1))
    x = x.reshape(-1)[: rng_blocks * B]
    codes, alpha32, s32 = oracle_mod.compress(x, B)
    g_rec = oracle_mod.reconstruct_f64(codes, alpha32, s32, B)
    for k in range(rng_blocks):
        xb = x[k * B:(k + 1) * B]
        a64, _, z = oracle_mod.ash_block(xb, B)
        s64 = np.max(np.abs(z)) / QMAX
        v = z / s64
        dec = oracle_mod.e4m3_decode(codes[k * B:(k + 1) * B])
        av = np.abs(v)
        e = np.floor(np.log2(np.maximum(av, 2.0 ** -6)))
        spacing = np.exp2(e - 3)
        assert np.all(np.abs(dec - v) <= 0.5 * spacing + 2.0 ** -24 * av + 1e-12)
        zhat = dec * float(s32[k])
        lhs = np.linalg.norm(g_rec[k * B:(k + 1) * B] - bits_to_f64(xb))
        rhs = np.linalg.norm(zhat / float(alpha32[k]) - z / a64)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9)


# ---------------------------------------------- output rounding ----------

def test_double_to_bf16_is_nearest_even(oracle_mod):
    import torch
    rng = np.random.default_rng(3)
    # Values exact in float32: must agree with torch's float32 -> bfloat16.
    f = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-130, 120, 200_000))).astype(np.float32)
    ours = oracle_mod.double_to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # Values between bf16 neighbours: the nearer neighbour, ties to even.
    d = rng.standard_normal(100_000) * np.exp2(rng.uniform(-20, 20, 100_000))
    got = bits_to_f64(oracle_mod.double_to_bf16(d))
    lo_bits = oracle_mod.double_to_bf16(d)
    for i in range(0, d.size, 997):
        v = d[i]
        b = int(lo_bits[i])
        nb = [b - 1, b, b + 1]
        cand = bits_to_f64(np.array(nb, np.uint16))
        best = np.min(np.abs(cand - v))
        assert abs(got[i] - v) == best


def test_accumulate_adds_float32_rounded_reconstruction(oracle_mod):
    import synth
    B = 128
    x = synth.generate(synth.WORKLOADS["laplace_2048x1024"].with_shape(8))
    codes, alpha, s = oracle_mod.compress(x, B)
    g = oracle_mod.reconstruct_f64(codes, alpha, s, B)
    acc = np.zeros(x.shape, np.float32)
    oracle_mod.decompress_accumulate(codes, alpha, s, B, acc)
    assert np.array_equal(acc, g.astype(np.float32))
    oracle_mod.decompress_accumulate(codes, alpha, s, B, acc)
    assert np.array_equal(acc, g.astype(np.float32) * np.float32(2))
    y = oracle_mod.decompress(codes, alpha, s, B)
    assert np.array_equal(y, oracle_mod.double_to_bf16(g))


def test_fidelity_is_sane_on_laplace_workload(oracle_mod):
    """Not a pinned level (the paper prints no operator-level error figure):
    a coarse guard that the whole chain reconstructs the tensor."""
    import synth
    x = synth.generate(synth.WORKLOADS["laplace_2048x1024"].with_shape(64))
    for B in (128, 256):
        codes, alpha, s = oracle_mod.compress(x, B)
        g = oracle_mod.reconstruct_f64(codes, alpha, s, B)
        xf = bits_to_f64(x)
        rel = np.linalg.norm(g - xf) / np.linalg.norm(xf)
        assert rel < 0.05, rel
