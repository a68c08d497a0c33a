"""The seeded input generator: deterministic, thread-count independent, and
drawing the distributions its recipes name."""
import numpy as np
import pytest


def test_deterministic_and_thread_independent(synth_mod):
    r = synth_mod.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(96)
    a = synth_mod.generate(r, threads=1)
    b = synth_mod.generate(r, threads=7)
    c = synth_mod.generate(r)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    d = synth_mod.generate(r, seed=r.seed + 1)
    assert np.mean(a != d) > 0.9


def test_rows_are_a_prefix_of_the_full_tensor(synth_mod):
    """Element values depend only on (seed, flattened index)."""
    r = synth_mod.WORKLOADS["laplace_2048x1024"]
    small = synth_mod.generate(r.with_shape(16))
    big = synth_mod.generate(r.with_shape(64))
    assert np.array_equal(big[:16], small)


def test_laplace_body_and_t_outliers(synth_mod):
    r = synth_mod.WORKLOADS["laplace_2048x1024"].with_shape(512)
    x = synth_mod.bits_to_f32(synth_mod.generate(r)).astype(np.float64)
    body = x[np.abs(x) < 0.5]
    # Laplace(0, b): E|x| = b.
    assert abs(np.mean(np.abs(body)) / 0.02 - 1) < 0.02
    assert abs(np.mean(x)) < 1e-3
    # 0.1% of entries are 0.5 * t3: most exceed the body's range.
    frac_big = np.mean(np.abs(x) > 0.3)
    assert 2e-4 < frac_big < 1.5e-3


def test_outlier_channels(synth_mod):
    r = synth_mod.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(256)
    x = synth_mod.bits_to_f32(synth_mod.generate(r)).astype(np.float64)
    cols = synth_mod.outlier_columns(r)
    assert len(set(cols.tolist())) == 4
    mag = np.mean(np.abs(x), axis=0)
    others = np.delete(mag, cols)
    assert np.allclose(mag[cols] / np.mean(others), 30.0, rtol=0.1)
    assert np.all(others < 2 * np.mean(others))


def test_gradient_zeros_and_mixture(synth_mod):
    g = synth_mod.WORKLOADS["grad_8192x8192"].with_shape(64)
    x = synth_mod.bits_to_f32(synth_mod.generate(g))
    assert abs(np.mean(x == 0) - 0.01) < 1e-3
    cols = synth_mod.outlier_columns(g)
    body = np.delete(x, cols, axis=1)
    assert abs(np.std(body[body != 0]) / 1e-4 - 1) < 0.02
    q = synth_mod.WORKLOADS["qwen7b_act_16384x3584"].with_shape(64)
    y = synth_mod.bits_to_f32(synth_mod.generate(q)).astype(np.float64)
    # Mixture variance: 0.95 * 0.005^2 + 0.05 * 0.1^2.
    assert abs(np.var(y) / (0.95 * 0.005 ** 2 + 0.05 * 0.1 ** 2) - 1) < 0.05


def test_bf16_bit_helpers_round_trip(synth_mod):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 10000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]        # finite only
    assert np.array_equal(synth_mod.f32_to_bits(synth_mod.bits_to_f32(bits)), bits)
