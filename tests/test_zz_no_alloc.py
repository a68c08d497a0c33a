"""taco_roundtrip_noalloc (the round trip for callers that cannot allocate)
against taco_roundtrip, through the C ABI, on the GPU.

Two calls in a row share the library's per-GPU working array; the second
has a smaller input (and a smaller tensor maximum), so anything the first
call left in the array would show in the second's totals.  Every case prints
its name before it touches the GPU.
"""
from __future__ import annotations

import struct

import numpy as np
import pytest

import oracle
import synth
from parity import rel_rms, RECON_RTOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def taco():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gradients_taco_compress_amd as taco
    return taco


def announce(msg):
    print(f"[case] {msg}", flush=True)


def totals_of(buf):
    """(sum_sq_err, sum_sq_ref, sum_sq_out, sum_dot, max_abs_err, tensor_absmax)
    from the first 40 bytes of a device buffer."""
    return struct.unpack("<4d2f", bytes(buf[:40].cpu().numpy().tobytes()))


def run_both(taco, x_bits, block, variant, fmt, tau=1.0):
    """One call of each entry point on the same input, through the C ABI.
    Returns (y, totals) of taco_roundtrip and of taco_roundtrip_noalloc."""
    import torch
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)
    tokens, hidden = x.shape
    f, v = taco.FORMATS[fmt], taco.VARIANTS[variant]
    stream = torch.cuda.current_stream().cuda_stream
    sums = torch.empty(taco.FIDELITY_SUMS_BYTES, dtype=torch.uint8, device="cuda")
    totals = torch.full((taco.FIDELITY_TOTALS_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    y_ref = torch.empty_like(x)
    y_new = torch.empty_like(x)
    st = taco.taco_roundtrip(x.data_ptr(), tokens, hidden, block, tau, f, v, y_ref.data_ptr(),
                             sums.data_ptr(), stream)
    assert st == 0, taco.taco_status_string(st)
    st = taco.taco_roundtrip_noalloc(x.data_ptr(), tokens, hidden, block, tau, f, v,
                                     y_new.data_ptr(), totals.data_ptr(), stream)
    assert st == 0, taco.taco_status_string(st)
    torch.cuda.synchronize()
    yb = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return (yb(y_ref), totals_of(sums)), (yb(y_new), totals_of(totals))


def check_pair(taco, x_bits, block, variant, fmt):
    (y_ref, t_ref), (y_new, t_new) = run_both(taco, x_bits, block, variant, fmt)
    # Same kernels on the same input: the reconstruction is bit-identical.
    assert np.array_equal(y_new, y_ref), f"{variant}/{fmt}: outputs differ"
    # The double totals are summed with atomics, whose order varies between
    # calls: equal to the last bits (1e-12 relative); the maxima exactly.
    for a, b, name in zip(t_new[:4], t_ref[:4], ("sum_sq_err", "sum_sq_ref", "sum_sq_out",
                                                 "sum_dot")):
        assert a == pytest.approx(b, rel=1e-12, abs=1e-300), (name, a, b)
    assert t_new[4] == t_ref[4], ("max_abs_err", t_new[4], t_ref[4])
    assert t_new[5] == t_ref[5], ("tensor_absmax", t_new[5], t_ref[5])
    # And both against the oracle's round trip of the same variant.
    xo = oracle.roundtrip_variant(x_bits, block, variant, fmt).reshape(-1)
    xo_bf16 = synth.bits_to_f32(oracle.double_to_bf16(xo)).astype(np.float64)
    r = rel_rms(synth.bits_to_f32(y_new).reshape(-1).astype(np.float64), xo_bf16)
    assert r <= RECON_RTOL, f"{variant}/{fmt}: reconstruction rel RMS {r:.3g} vs the oracle"
    ref = synth.bits_to_f32(x_bits).astype(np.float64).reshape(-1)
    assert t_new[1] == pytest.approx(float(np.dot(ref, ref)), rel=1e-6)
    if variant == "tensor":
        assert t_new[5] == float(np.max(np.abs(ref)))
    return t_new


@pytest.mark.parametrize("variant,fmt,block", [("taco", "e4m3", 128), ("tensor", "int8", 256),
                                               ("ds", "e5m2", 64)])
def test_noalloc_matches_roundtrip_on_two_calls(taco, variant, fmt, block):
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"]
    # First call: 1024 x 2560 with the workload's outlier channels, times 4
    # (exact in bf16), so that its maximum exceeds the second input's.
    big = synth.f32_to_bits(4.0 * synth.bits_to_f32(synth.generate(r.with_shape(1024, seed=61))))
    announce(f"noalloc {variant}/{fmt} B={block} first call 1024x2560")
    t1 = check_pair(taco, big, block, variant, fmt)
    # Second call: a smaller tensor (37 x 1536, a ragged last wave-step) with a
    # smaller maximum, so stale sums or a stale maximum would be visible.
    small = synth.generate(synth.WORKLOADS["laplace_2048x1024"].with_shape(37, 1536, seed=62))
    announce(f"noalloc {variant}/{fmt} B={block} second call 37x1536")
    t2 = check_pair(taco, small, block, variant, fmt)
    assert t2[1] < t1[1]
    if variant == "tensor":          # tensor_absmax is written by that variant only
        assert t2[5] < t1[5]


def test_noalloc_empty_is_a_noop(taco):
    import torch
    announce("noalloc empty tensor")
    totals = torch.full((taco.FIDELITY_TOTALS_BYTES,), 7, dtype=torch.uint8, device="cuda")
    st = taco.taco_roundtrip_noalloc(0, 0, 1024, 128, 1.0, 0, 0, 0, totals.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.all(totals == 7)
