"""Parity of the fused owner step (taco_reduce_compress) with the oracle, on
the GPU, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import compare_reduce

pytestmark = pytest.mark.gpu


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


def gpu_payloads(taco, xs, B):
    """Compress each bf16 array on the GPU; return (gpu tuples, numpy tuples)."""
    g, h = [], []
    for x in xs:
        c, a, s = taco.compress(to_gpu_bf16(x), block=B)
        g.append((c, a, s))
        h.append((c.cpu().numpy(), a.cpu().numpy(), s.cpu().numpy()))
    return g, h


def run_case(taco, own_bits, xs, B, tau=1.0, cancelling=False):
    import torch
    pay_g, pay_h = gpu_payloads(taco, xs, B)
    own = None if own_bits is None else to_gpu_bf16(own_bits)
    codes, alpha, scale = taco.reduce_compress(own, pay_g, block=B, target_energy=tau)
    torch.cuda.synchronize()
    return compare_reduce(own_bits, pay_h, B, codes.cpu().numpy(), alpha.cpu().numpy(),
                          scale.cpu().numpy(), tau, cancelling=cancelling)


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("P", [0, 1, 3, 7, 8])
def test_ragged_all_blocks_and_payload_counts(taco, B, P):
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(37, 1536)
    announce(f"owner step 37x1536 B={B} P={P}")
    own = synth.generate(r, seed=100)
    xs = [synth.generate(r, seed=101 + p) for p in range(P)]
    print(run_case(taco, own, xs, B), flush=True)


@pytest.mark.parametrize("B", [128, 256])
def test_without_own_partial(taco, B):
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(16, 3584)
    announce(f"owner step, no own partial, B={B}")
    xs = [synth.generate(r, seed=200 + p) for p in range(3)]
    run_case(taco, None, xs, B)


@pytest.mark.parametrize("B", [32, 128, 512])
def test_cancelling_and_special_sums(taco, B):
    """own = x and a payload compressed from -x leave only the quantisation
    error; constant blocks sum exactly; huge values exercise the rescaled
    energy branch, up to the top of the bf16 range.  B = 32, 128 and 512
    cover the three lane layouts (4, 8 and 16 lanes per block)."""
    rng = np.random.default_rng(3)
    x = synth.f32_to_bits(rng.laplace(0, 0.02, 16 * B))
    neg = x ^ np.uint16(0x8000)
    announce(f"owner step special sums B={B}")
    st = run_case(taco, x, [neg], B, cancelling=True)
    print(f"cancelling sum: {st['flips']} flips in {st['n']} elements, all at ties within "
          f"the float32 bound", flush=True)
    const = synth.f32_to_bits(np.repeat(rng.uniform(-2, 2, 16), B))
    run_case(taco, const, [const, const], B)
    huge = synth.f32_to_bits(rng.standard_normal(16 * B) * 1e30)
    run_case(taco, huge, [huge], B)
    zero = np.zeros(16 * B, np.uint16)
    run_case(taco, zero, [x], B)
    # Tiny blocks (bf16 subnormals, 1e-37 normals): rotated values and
    # payload factors below the float32 normals.
    sub = rng.integers(1, 0x7F, 16 * B).astype(np.uint16) | (rng.integers(0, 2, 16 * B).astype(np.uint16) << 15)
    tiny = synth.f32_to_bits(rng.standard_normal(16 * B) * 1e-37)
    tiny2 = synth.f32_to_bits(rng.standard_normal(16 * B) * 3e-38)
    run_case(taco, None, [tiny, tiny2, sub], B)
    run_case(taco, sub, [sub, tiny], B)
    # Top of the bf16 range, where H X (B |X|) leaves float32 range.
    top = synth.f32_to_bits(np.clip(rng.standard_normal(16 * B) * 5e37, -2.5e38, 2.5e38))
    run_case(taco, top, [top], B)
    run_case(taco, None, [top, top], B)


def test_tau_scales_alpha_and_s(taco):
    r = synth.WORKLOADS["grad_8192x8192"].with_shape(4, 8192)
    own = synth.generate(r, seed=300)
    xs = [synth.generate(r, seed=301 + p) for p in range(2)]
    announce("owner step tau")
    for tau in (0.5, 37.5):
        run_case(taco, own, xs, 256, tau)


def test_owner_step_at_workload_scale(taco):
    """The 32768x12288 workload: own partial plus three received payloads
    (four independently seeded tensors), every block against the oracle."""
    import torch
    name, B = "gpt175b_hidden_32768x12288", 256
    r = synth.WORKLOADS[name]
    seeds = synth.ACCUMULATE_SEEDS
    announce(f"owner step {name} P=3 (full)")
    own_bits = synth.generate(r, seed=seeds[0])
    pay = []
    for sd in seeds[1:]:
        xg = to_gpu_bf16(synth.generate(r, seed=sd))
        pay.append(taco.compress(xg, block=B))
        del xg
    codes, alpha, scale = taco.reduce_compress(to_gpu_bf16(own_bits), pay, block=B)
    torch.cuda.synchronize()
    pay_h = [(c.cpu().numpy(), a.cpu().numpy(), s.cpu().numpy()) for c, a, s in pay]
    del pay
    st = compare_reduce(own_bits, pay_h, B, codes.cpu().numpy(), alpha.cpu().numpy(),
                        scale.cpu().numpy())
    print(st, flush=True)
