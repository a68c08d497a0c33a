"""Several payloads into one float32 accumulator in one pass
(taco_decompress_accumulate_n), on the GPU through the C ABI, against the
oracle (decompress_accumulate_n) and against one accumulate per payload.

Every case prints its name before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import compare_accumulate_n, rel_rms

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


def to_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def payloads(taco, xs, B, fmt="e4m3"):
    g, h = [], []
    for x in xs:
        c, a, s = taco.compress(to_gpu_bf16(x), block=B, fmt=fmt)
        g.append((c, a, s))
        h.append((c.cpu().numpy().reshape(-1), a.cpu().numpy(), s.cpu().numpy()))
    return g, h


def check(taco, xs, B, acc0, fmt="e4m3"):
    import torch
    g, h = payloads(taco, xs, B, fmt)
    acc = to_gpu(acc0.copy())
    taco.decompress_accumulate_n(g, acc, block=B, fmt=fmt)
    seq = to_gpu(acc0.copy())
    for c, a, s in g:
        taco.decompress_accumulate(c, a, s, seq, block=B, fmt=fmt)
    torch.cuda.synchronize()
    got = acc.cpu().numpy().reshape(-1)
    want = oracle.decompress_accumulate_n(h, B, acc0.copy().reshape(-1), fmt)
    r = rel_rms(got, want)
    assert r <= 1e-6, f"vs oracle rel RMS {r:.3g}"
    r2 = rel_rms(got, seq.cpu().numpy().reshape(-1))
    assert r2 <= 1e-6, f"vs sequential accumulates rel RMS {r2:.3g}"
    # Element-wise: within the (worst-case) float32 bound of the
    # rotated-domain sum, and within 2^-20 of the block's magnitude (a
    # tighter bound that holds in practice: the rounding errors do not line
    # up with one Walsh row).
    st = compare_accumulate_n(got, acc0, h, B, fmt)
    assert st["max_err_over_block_magnitude"] <= 2.0 ** -20, st
    return r, r2


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_all_blocks_and_payload_counts(taco, B, P):
    r = synth.WORKLOADS["gpt175b_hidden_32768x12288"].with_shape(37, 1536)
    announce(f"accumulate_n 37x1536 B={B} P={P}")
    xs = [synth.generate(r, seed=600 + p) for p in range(P)]
    acc0 = synth.bits_to_f32(synth.generate(r, seed=699)).astype(np.float32)
    print(check(taco, xs, B, acc0), flush=True)


@pytest.mark.parametrize("fmt", ["e5m2", "int8"])
def test_formats(taco, fmt):
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(8, 3584)
    announce(f"accumulate_n {fmt} 8x3584 B=256 P=3")
    xs = [synth.generate(r, seed=610 + p) for p in range(3)]
    check(taco, xs, 256, np.zeros(8 * 3584, np.float32), fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
def test_packed_equals_side(taco, fmt):
    import torch
    r = synth.WORKLOADS["grad_8192x8192"].with_shape(4, 8192)
    announce(f"accumulate_n packed {fmt} 4x8192 B=256 P=4")
    xs = [to_gpu_bf16(synth.generate(r, seed=620 + p)) for p in range(4)]
    side = [taco.compress(x, block=256, fmt=fmt) for x in xs]
    packed = [taco.compress_packed(x, block=256, fmt=fmt) for x in xs]
    a1 = torch.zeros((4, 8192), dtype=torch.float32, device="cuda")
    a2 = torch.zeros_like(a1)
    taco.decompress_accumulate_n(side, a1, block=256, fmt=fmt)
    taco.decompress_accumulate_n_packed(packed, a2, block=256, fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2)


def test_special_blocks(taco):
    """Zero, tiny, huge and bf16-maximum blocks (the shifted sums)."""
    from test_gpu_parity import special_blocks
    for B in (32, 128, 512):                 # 4, 8 and 16 lanes per block
        x = special_blocks(B)
        announce(f"accumulate_n special blocks B={B}")
        g, h = payloads(taco, [x], B)
        flipped = x ^ np.uint16(0x8000)          # the same blocks negated
        g2, h2 = payloads(taco, [flipped], B)
        acc = to_gpu(np.zeros(x.size, np.float32))
        taco.decompress_accumulate_n(g + g2, acc, block=B)
        got = acc.cpu().numpy().reshape(-1, B)
        want = oracle.decompress_accumulate_n(h + h2, B, np.zeros(x.size, np.float32)).reshape(-1, B)
        mag = (np.abs(oracle.reconstruct_f64(*h[0], B)) +
               np.abs(oracle.reconstruct_f64(*h2[0], B))).reshape(-1, B)
        for k in range(x.shape[0]):
            # x and -x: the exact sum is 0 up to each payload's own rounding.
            tol = 2.0 ** -20 * np.max(mag[k]) + 1e-37
            assert np.all(np.abs(got[k] - want[k]) <= tol), (B, k)
        acc1 = to_gpu(np.zeros(x.size, np.float32))
        taco.decompress_accumulate_n(g, acc1, block=B)
        want1 = oracle.decompress_accumulate_n(h, B, np.zeros(x.size, np.float32)).reshape(-1, B)
        got1 = acc1.cpu().numpy().reshape(-1, B)
        for k in range(x.shape[0]):
            if np.any(want1[k] != 0):
                assert rel_rms(got1[k], want1[k]) <= 1e-6, (B, k)
            else:
                assert np.all(got1[k] == 0), (B, k)


def test_workload_scale_four_payloads(taco):
    """The 32768x12288 workload: four payloads into one accumulator in one
    pass, every element against the oracle (within the float32 bound of the
    rotated-domain sum) and the relative RMS."""
    import torch
    name, B = "gpt175b_hidden_32768x12288", 256
    r = synth.WORKLOADS[name]
    g, h = [], []
    for seed in synth.ACCUMULATE_SEEDS:
        announce(f"accumulate_n workload payload seed={seed}")
        x = to_gpu_bf16(synth.generate(r, seed=seed))
        c, a, s = taco.compress(x, block=B)
        del x
        g.append((c, a, s))
        h.append((c.cpu().numpy().reshape(-1), a.cpu().numpy(), s.cpu().numpy()))
    acc = torch.zeros((r.rows, r.cols), dtype=torch.float32, device="cuda")
    taco.decompress_accumulate_n(g, acc, block=B)
    torch.cuda.synchronize()
    announce("accumulate_n workload vs the oracle (full)")
    st = compare_accumulate_n(acc.cpu().numpy(), np.zeros(r.numel, np.float32), h, B)
    print(st, flush=True)
    assert st["max_err_over_block_magnitude"] <= 2.0 ** -20, st
