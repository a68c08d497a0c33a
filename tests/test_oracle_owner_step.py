"""Pins of the oracle's owner step of the two-shot all-reduce (TACO paper,
section 4.4.2: the reduce-scatter phase ends in one local reduction of the
received payloads; the reduced segment is compressed again for the
all-gather), built from Eq. 11-13, a sum, and Eq. 5-10.

Pinned against: its two degenerate cases (no payloads; no own partial),
which reduce to the already-pinned compress; closed forms for blocks whose
payloads reconstruct exactly (constant blocks, spikes plus Walsh rows); and
invariance under reordering the payloads.  The multi-payload accumulate
(the same local reduction into a float32 accumulator) is pinned by its one-
and zero-payload cases and by the exactly rounded sum of reconstructions.
"""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

import synth

EPS = 1e-20
QMAX = 448.0


def f32_to_bits(v):
    import synth
    return synth.f32_to_bits(np.asarray(v, np.float32))


def bits_to_f64(bits):
    import synth
    return synth.bits_to_f32(bits).astype(np.float64)


@pytest.fixture(scope="module")
def workload_blocks(synth_mod):
    r = synth_mod.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(4, 2560)
    return [synth_mod.generate(r, seed=s) for s in (40, 41, 42, 43)]


@pytest.mark.parametrize("B", [128, 256])
def test_degenerate_cases_reduce_to_compress(oracle_mod, workload_blocks, B):
    own = workload_blocks[0]
    assert all(np.array_equal(a, b) for a, b in
               zip(oracle_mod.reduce_compress(own, [], B), oracle_mod.compress(own, B)))
    pay = oracle_mod.compress(workload_blocks[1], B)
    g = oracle_mod.reconstruct_f64(*pay, B)
    assert all(np.array_equal(a, b) for a, b in
               zip(oracle_mod.reduce_compress(None, [pay], B), oracle_mod.compress_f64(g, B)))


@pytest.mark.parametrize("B", [32, 128, 512])
def test_constant_blocks_sum_exactly(oracle_mod, B):
    """Constant blocks reconstruct exactly, so own c0 plus payloads c1, c2
    reduce to the constant c0 + c1 + c2: one code at +-Q_max."""
    for c0, c1, c2 in [(0.5, 0.25, -0.125), (-3.0, 1.0, 1.5), (1e-3, -2e-3, -5e-4)]:
        own = f32_to_bits(np.full(B, c0))
        p1 = oracle_mod.compress(f32_to_bits(np.full(B, c1)), B)
        p2 = oracle_mod.compress(f32_to_bits(np.full(B, c2)), B)
        total = sum(float(bits_to_f64(f32_to_bits([c]))[0]) for c in (c0, c1, c2))
        codes, alpha, scale = oracle_mod.reduce_compress(own, [p1, p2], B)
        want = np.zeros(B, np.uint8)
        want[0] = 0x7E if total > 0 else 0xFE
        assert np.array_equal(codes, want)
        a = 1.0 / math.sqrt(total * total + EPS)
        np.testing.assert_allclose(alpha[0], a, rtol=1e-7)
        np.testing.assert_allclose(scale[0], a * abs(total) * math.sqrt(B) / QMAX, rtol=1e-6)


@pytest.mark.parametrize("B", [64, 256])
def test_spike_plus_walsh_row(oracle_mod, B):
    """own = a e_p and a payload b H[r, :] (exact reconstruction) give
    Z_j = alpha (a H[j, p] + b B delta_jr) / sqrt(B) in closed form."""
    H = hadamard(B).astype(np.float64)
    for p, r, a, b in [(3, 5, 0.75, 0.125), (B - 1, 0, -2.0, 0.5), (7, B // 2, 1.0, -0.0078125)]:
        own_v = np.zeros(B)
        own_v[p] = a
        pay = oracle_mod.compress(f32_to_bits(b * H[r]), B)
        codes, alpha, scale = oracle_mod.reduce_compress(f32_to_bits(own_v), [pay], B)
        x = own_v + b * H[r]
        al = 1.0 / math.sqrt(np.mean(x ** 2) + EPS)
        z = al * (a * H[:, p] + b * B * (np.arange(B) == r)) / math.sqrt(B)
        s = np.max(np.abs(z)) / QMAX
        want = oracle_mod.e4m3_encode((z / s).astype(np.float32))
        assert np.array_equal(codes, want)
        np.testing.assert_allclose(alpha[0], al, rtol=1e-7)
        np.testing.assert_allclose(scale[0], s, rtol=1e-7)


def test_payload_order_does_not_matter(oracle_mod, workload_blocks):
    B = 128
    pays = [oracle_mod.compress(x, B) for x in workload_blocks[1:]]
    c1, a1, s1 = oracle_mod.reduce_compress(workload_blocks[0], pays, B)
    c2, a2, s2 = oracle_mod.reduce_compress(workload_blocks[0], pays[::-1], B)
    assert np.count_nonzero(c1 != c2) <= 2          # double rounding order only
    np.testing.assert_allclose(a1, a2, rtol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12)


# ------------------------------------------- several payloads at once ----

def _payloads(oracle_mod, P, B, fmt="e4m3", seed=90):
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(3, 1024, seed=seed)
    return [oracle_mod.compress(synth.generate(r, seed=seed + p), B, fmt=fmt) for p in range(P)]


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
def test_accumulate_n_of_one_payload_is_accumulate(oracle_mod, fmt):
    pay = _payloads(oracle_mod, 1, 128, fmt)
    acc0 = synth.bits_to_f32(synth.generate(synth.WORKLOADS["laplace_2048x1024"].with_shape(3, 1024, seed=7)))
    acc0 = acc0.astype(np.float32).reshape(-1)
    a = oracle_mod.decompress_accumulate_n(pay, 128, acc0.copy(), fmt)
    b = oracle_mod.decompress_accumulate(*pay[0], 128, acc0.copy(), fmt=fmt)
    assert np.array_equal(a, b)


def test_accumulate_n_of_nothing_is_a_no_op(oracle_mod):
    acc = np.arange(3 * 1024, dtype=np.float32)
    out = oracle_mod.decompress_accumulate_n([], 128, acc.copy())
    assert np.array_equal(out, acc)


def test_accumulate_n_is_the_rounded_exact_sum(oracle_mod):
    """The payloads' exact reconstructions, summed, rounded once: a payload
    repeated twice adds exactly twice its reconstruction (x2 is exact), and
    several payloads agree with sequential accumulation to float32 rounding."""
    pay = _payloads(oracle_mod, 3, 256)
    g = [oracle_mod.reconstruct_f64(*p, 256) for p in pay]
    zero = np.zeros(3 * 1024, np.float32)
    twice = oracle_mod.decompress_accumulate_n([pay[0], pay[0]], 256, zero.copy())
    assert np.array_equal(twice, (2.0 * g[0]).astype(np.float32).reshape(-1))
    fused = oracle_mod.decompress_accumulate_n(pay, 256, zero.copy())
    want = (g[0] + g[1] + g[2]).astype(np.float32).reshape(-1)
    assert np.array_equal(fused, want)
    seq = zero.copy()
    for p in pay:
        oracle_mod.decompress_accumulate(*p, 256, seq)
    scale = np.abs(g[0]) + np.abs(g[1]) + np.abs(g[2])
    assert np.all(np.abs(seq - fused) <= 4 * 2.0 ** -24 * scale.reshape(-1) + 1e-45)
