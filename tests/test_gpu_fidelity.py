"""The fidelity study on the GPU (taco_roundtrip, through the C ABI): every
variant's round trip and its error sums against the oracle's
(roundtrip_variant, fidelity), for every code format.

Every case prints its name before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import compare_roundtrip, rel_rms, RECON_RTOL

pytestmark = pytest.mark.gpu

VARIANTS = ["taco", "direct", "ds", "ash", "hadamard", "tensor"]
FORMATS = ["e4m3", "e5m2", "int8"]


@pytest.fixture(scope="module")
def taco():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gradients_taco_compress_amd as taco
    return taco


def announce(msg):
    print(f"[case] {msg}", flush=True)


def to_gpu_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bf16_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_variant(taco, x_bits, B, variant, fmt, tau=1.0):
    """GPU round trip (y and sums) against the oracle's x' and metrics."""
    x = to_gpu_bf16(x_bits)
    y, sums = taco.roundtrip(x, block=B, variant=variant, fmt=fmt, target_energy=tau,
                             want_output=True)
    n = x_bits.size
    m = taco.fidelity_metrics(sums, n)
    ref = synth.bits_to_f32(x_bits).astype(np.float64).reshape(-1)
    xo = oracle.roundtrip_variant(x_bits, B, variant, fmt, tau).reshape(-1)
    mo = oracle.fidelity(ref, xo)
    # Reconstruction: every element against the oracle's x' (one bf16
    # rounding plus the float32 error of the kernel, tie flips explained as
    # adjacent-code changes), and the relative RMS against the oracle's x'
    # rounded to bf16 as the GPU's output is.
    compare_roundtrip(bf16_bits(y), x_bits, B, variant, fmt, tau, xo=xo)
    # Sums: the reference energy exactly as the oracle's up to float32
    # partial sums; the error metrics to the reconstruction tolerance.
    assert m["sum_sq_ref"] == pytest.approx(float(np.dot(ref, ref)), rel=1e-6)
    if mo["rel_l2"] > 0:
        assert m["rel_l2"] == pytest.approx(mo["rel_l2"], rel=RECON_RTOL), (m, mo)
        assert m["mse"] == pytest.approx(mo["mse"], rel=2 * RECON_RTOL), (m, mo)
    else:
        assert m["rel_l2"] <= 1e-6
    assert m["cos"] == pytest.approx(mo["cos"], abs=1e-6), (m, mo)
    # A flip at a rounding tie leaves that element's error unchanged, so the
    # maximum error agrees up to float32 rounding.
    assert m["max_err"] == pytest.approx(mo["max_err"], rel=1e-4, abs=1e-30), (m, mo)
    if variant == "tensor":
        assert m["tensor_absmax"] == float(np.max(np.abs(ref)))
    return m, mo


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_matches_oracle(taco, variant, fmt):
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(37, 1536, seed=14)
    announce(f"roundtrip {variant}/{fmt} 37x1536 B=128")
    m, mo = check_variant(taco, synth.generate(r), 128, variant, fmt)
    print(variant, fmt, {k: m[k] for k in ("rel_l2", "cos", "max_err", "mse")}, flush=True)


@pytest.mark.parametrize("B", [32, 64, 256, 512])
@pytest.mark.parametrize("variant", ["taco", "ds", "ash", "hadamard"])
def test_block_sizes(taco, variant, B):
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(5, 3584, seed=15)
    announce(f"roundtrip {variant}/e4m3 5x3584 B={B}")
    check_variant(taco, synth.generate(r), B, variant, "e4m3")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("B", [32, 128, 512])
def test_taco_variant_equals_compress_then_decompress(taco, fmt, B):
    """The fused round trip repeats the operator's arithmetic exactly."""
    import torch
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(41, 2560, seed=16)
    announce(f"roundtrip == compress+decompress {fmt} 41x2560 B={B}")
    x = to_gpu_bf16(synth.generate(r))
    y, _ = taco.roundtrip(x, block=B, variant="taco", fmt=fmt, want_output=True)
    c, a, s = taco.compress(x, block=B, fmt=fmt)
    y2 = taco.decompress(c, a, s, block=B, fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("B", [32, 128, 512])
@pytest.mark.parametrize("variant", VARIANTS)
def test_special_blocks(taco, variant, B):
    """The rare branches (huge and tiny blocks, zeros, subnormals) in every
    variant, in the three lane layouts (4, 8 and 16 lanes per block)."""
    from test_gpu_parity import special_blocks
    x = special_blocks(B)
    announce(f"roundtrip {variant} special blocks B={B}")
    xg = to_gpu_bf16(x)
    y, sums = taco.roundtrip(xg, block=B, variant=variant, want_output=True)
    xo = oracle.roundtrip_variant(x, B, variant).reshape(x.shape)
    want = synth.bits_to_f32(oracle.double_to_bf16(xo)).astype(np.float64)
    got = synth.bits_to_f32(bf16_bits(y)).astype(np.float64)
    for k in range(x.shape[0]):
        assert rel_rms(got[k], want[k]) <= RECON_RTOL, (variant, k)
    compare_roundtrip(bf16_bits(y), x, B, variant, "e4m3", xo=xo.reshape(-1))


def test_tensor_scale_sees_the_whole_tensor(taco):
    """The per-tensor maximum lives in the last block: every block's step
    follows it."""
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(16, 1024, seed=17)
    x = synth.generate(r)
    x[-1, -1] = synth.f32_to_bits(np.array([-37.0]))[0]
    announce("roundtrip tensor, max in the last element")
    for fmt in FORMATS:
        check_variant(taco, x, 256, "tensor", fmt)


def test_empty_and_no_output(taco):
    import torch
    announce("roundtrip empty / sums only")
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    y, sums = taco.roundtrip(x, block=128)
    assert y is None
    r = synth.WORKLOADS["grad_8192x8192"].with_shape(8, 8192, seed=18)
    xb = synth.generate(r)
    _, s1 = taco.roundtrip(to_gpu_bf16(xb), block=256)
    m1 = taco.fidelity_metrics(s1, xb.size)
    m2, _ = check_variant(taco, xb, 256, "taco", "e4m3")
    assert m1["rel_l2"] == pytest.approx(m2["rel_l2"], rel=1e-9)


@pytest.mark.parametrize("name,B", [("gpt2.7b_rowpar_8192x2560", 128), ("grad_8192x8192", 256)])
def test_full_size_sums(taco, name, B):
    """Full-size tensors: the GPU's sums against the oracle's on the whole
    tensor for the operator and its two scale-only variants."""
    r = synth.WORKLOADS[name]
    x_bits = synth.generate(r)
    x = to_gpu_bf16(x_bits)
    ref = synth.bits_to_f32(x_bits).astype(np.float64).reshape(-1)
    for variant in ("taco", "ds", "tensor"):
        announce(f"roundtrip {variant} full {name} B={B}")
        _, sums = taco.roundtrip(x, block=B, variant=variant)
        m = taco.fidelity_metrics(sums, x_bits.size)
        mo = oracle.fidelity(ref, oracle.roundtrip_variant(x_bits, B, variant).reshape(-1))
        assert m["rel_l2"] == pytest.approx(mo["rel_l2"], rel=RECON_RTOL), (variant, m, mo)
        assert m["cos"] == pytest.approx(mo["cos"], abs=1e-6), (variant, m, mo)
        assert m["max_err"] == pytest.approx(mo["max_err"], rel=1e-4), (variant, m, mo)
        print(name, variant, {k: m[k] for k in ("rel_l2", "cos", "max_err", "mse")}, flush=True)
