"""The interleaved wire layout on the GPU (through the C ABI): every packed
entry point must produce exactly what its side-buffer counterpart produces,
laid out as the oracle's pack() lays it out, and match the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import compare_compress, compare_decompress, compare_reduce, rel_rms

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


@pytest.mark.parametrize("B,rows,cols", [(32, 37, 1536), (64, 37, 1536), (128, 37, 1536),
                                          (256, 37, 1536), (512, 37, 1536),
                                          # two wave-steps per wave, odd count, partial tail
                                          (64, 131091, 64), (32, 262181, 32)])
def test_packed_equals_side_buffers_and_oracle(taco, B, rows, cols):
    import torch
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(rows, cols, seed=12)
    x_bits = synth.generate(r)
    announce(f"packed {rows}x{cols} B={B}")
    x = to_gpu_bf16(x_bits)
    c, a, s = taco.compress(x, block=B)
    pay = taco.compress_packed(x, block=B)
    torch.cuda.synchronize()
    pc, pa, ps = oracle.unpack(pay.cpu().numpy(), B)
    assert np.array_equal(pc, c.cpu().numpy().reshape(-1))
    assert np.array_equal(pa, a.cpu().numpy()) and np.array_equal(ps, s.cpu().numpy())
    compare_compress(x_bits, B, pc, pa, ps)
    # Receive side on the oracle's payload, packed by the oracle.
    oc, oa, os_ = oracle.compress(x_bits, B)
    opay = to_gpu(oracle.pack(oc, oa, os_, B).reshape(-1))
    y = taco.decompress_packed(opay, x.shape, block=B)
    y_side = taco.decompress(to_gpu(oc), to_gpu(oa), to_gpu(os_), block=B)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_side.view(torch.int16))
    compare_decompress(y.view(torch.int16).cpu().numpy().view(np.uint16), oc, oa, os_, B)
    acc = torch.zeros(x.shape, dtype=torch.float32, device="cuda")
    acc_side = torch.zeros_like(acc)
    taco.decompress_accumulate_packed(opay, acc, block=B)
    taco.decompress_accumulate(to_gpu(oc), to_gpu(oa), to_gpu(os_), acc_side, block=B)
    torch.cuda.synchronize()
    assert torch.equal(acc, acc_side)
    ref = oracle.decompress_accumulate(oc, oa, os_, B, np.zeros(x_bits.size, np.float32))
    assert rel_rms(acc.cpu().numpy().reshape(-1), ref) <= 1e-6


@pytest.mark.parametrize("B", [128, 256])
@pytest.mark.parametrize("P", [1, 3])
def test_packed_owner_step(taco, B, P):
    import torch
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(8, 3584)
    own_bits = synth.generate(r, seed=500)
    xs = [synth.generate(r, seed=501 + p) for p in range(P)]
    announce(f"packed owner step B={B} P={P}")
    own = to_gpu_bf16(own_bits)
    side = [taco.compress(to_gpu_bf16(v), block=B) for v in xs]
    packed = [taco.compress_packed(to_gpu_bf16(v), block=B) for v in xs]
    out_side = taco.reduce_compress(own, side, block=B)
    out_pack = taco.reduce_compress_packed(own, packed, block=B)
    torch.cuda.synchronize()
    uc, ua, us = oracle.unpack(out_pack.cpu().numpy(), B)
    assert np.array_equal(uc, out_side[0].cpu().numpy().reshape(-1))
    assert np.array_equal(ua, out_side[1].cpu().numpy())
    assert np.array_equal(us, out_side[2].cpu().numpy())
    pay_h = [oracle.unpack(p.cpu().numpy(), B) for p in packed]
    compare_reduce(own_bits, pay_h, B, uc, ua, us)
