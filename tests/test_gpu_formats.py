"""The E5M2 and INT8 code formats on the GPU, through the C ABI: the
conversions against the oracle's over every float32 inside their contracts,
and every operator entry point (compress, decompress, accumulate, owner step,
both layouts) against the oracle, as for E4M3.

Every case prints its name, format, shape and block before it touches the GPU.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
import synth
from conftest import build_helper, cpu_threads
from parity import compare_compress, compare_decompress, compare_reduce, rel_rms, RECON_RTOL

pytestmark = pytest.mark.gpu

FMTS = ["e5m2", "int8"]
# Largest magnitude (exclusive) inside each encoder's contract.
LIMIT = {"e5m2": 61440.0, "int8": 127.5}


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


def bf16_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------- codec ------

@pytest.mark.parametrize("fmt", FMTS)
def test_encode_matches_oracle_on_every_float_in_contract(taco, fmt):
    import torch
    helper = ctypes.CDLL(build_helper("encode_patterns"))
    helper.encode_pattern_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int]
    enc = oracle.encode_function_address(fmt)
    limit = int(np.array([LIMIT[fmt]], np.float32).view(np.uint32)[0])
    chunk = 1 << 26
    announce(f"{fmt} encode sweep over {2 * limit} patterns")
    for sign in (0, 1 << 31):
        for lo in range(0, limit, chunk):
            hi = min(lo + chunk, limit)
            pat = torch.arange(lo, hi, dtype=torch.int64, device="cuda").to(torch.int32)
            if sign:
                pat = pat | torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")
            got = taco.encode(pat.view(torch.float32), fmt).cpu().numpy()
            want = np.empty(hi - lo, np.uint8)
            helper.encode_pattern_range(lo | sign, hi | sign, enc,
                                        want.ctypes.data_as(ctypes.c_void_p), cpu_threads())
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (f"pattern {(lo | sign) + int(bad[0]):#010x}: gpu {got[bad[0]]:#x} "
                                   f"oracle {want[bad[0]]:#x} ({bad.size} mismatches)")


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_codes(taco, fmt):
    import torch
    announce(f"{fmt} decode all codes")
    codes = torch.arange(256, dtype=torch.int32, device="cuda").to(torch.uint8)
    got = taco.decode(codes, fmt).cpu().numpy().astype(np.float64)
    want = oracle.decode(np.arange(256, dtype=np.uint8), fmt)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


# ---------------------------------------------------------- operator ------

def full_check(taco, x_bits, B, fmt, tau=1.0):
    """GPU compress vs oracle; GPU decompress and accumulate of the oracle's
    payload vs the oracle; GPU round trip vs the oracle's round trip."""
    import torch
    x = to_gpu_bf16(x_bits)
    codes, alpha, scale = taco.compress(x, block=B, target_energy=tau, fmt=fmt)
    torch.cuda.synchronize()
    st = compare_compress(x_bits, B, codes.cpu().numpy(), alpha.cpu().numpy(),
                          scale.cpu().numpy(), tau, fmt=fmt)
    o_c, o_a, o_s = st.pop("oracle")
    shape = x_bits.shape
    y = taco.decompress(to_gpu(o_c.reshape(shape)), to_gpu(o_a), to_gpu(o_s), block=B, fmt=fmt)
    compare_decompress(bf16_bits(y), o_c, o_a, o_s, B, fmt=fmt)
    acc0 = synth.bits_to_f32(x_bits).astype(np.float32).reshape(shape)
    acc = to_gpu(acc0.copy())
    taco.decompress_accumulate(to_gpu(o_c.reshape(shape)), to_gpu(o_a), to_gpu(o_s), acc,
                               block=B, fmt=fmt)
    ref_acc = oracle.decompress_accumulate(o_c, o_a, o_s, B, acc0.copy().reshape(-1), fmt=fmt)
    r_acc = rel_rms(acc.cpu().numpy().reshape(-1), ref_acc)
    assert r_acc <= 1e-6, f"accumulate rel RMS {r_acc:.3g}"
    y2 = taco.decompress(codes, alpha, scale, block=B, fmt=fmt)
    torch.cuda.synchronize()
    ref = synth.bits_to_f32(oracle.decompress(o_c, o_a, o_s, B, fmt=fmt)).astype(np.float64)
    r = rel_rms(synth.bits_to_f32(bf16_bits(y2)).reshape(-1), ref.reshape(-1))
    assert r <= RECON_RTOL, f"round trip rel RMS vs oracle {r:.3g}"
    st.update(acc_rel=r_acc, roundtrip_rel=r)
    return st


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
def test_ragged_all_block_sizes(taco, fmt, B):
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(37, 1536, seed=13)
    announce(f"{fmt} ragged 37x1536 B={B}")
    print(full_check(taco, synth.generate(r), B, fmt), flush=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("tokens,hidden,B", [(131091, 64, 64), (262181, 32, 32)])
def test_paired_wave_steps(taco, fmt, tokens, hidden, B):
    # Two wave-steps per wave (B <= 64, at least 16384 wave-steps), an odd
    # count of them and a partial last one.
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(tokens, hidden, seed=43)
    announce(f"{fmt} paired wave-steps {tokens}x{hidden} B={B}")
    print(full_check(taco, synth.generate(r), B, fmt), flush=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [32, 256])
def test_special_blocks(taco, fmt, B):
    from test_gpu_parity import special_blocks
    x = special_blocks(B)
    announce(f"{fmt} special blocks B={B} ({x.shape[0]} blocks)")
    codes, alpha, scale = taco.compress(to_gpu_bf16(x), block=B, fmt=fmt)
    o_c, o_a, o_s = oracle.compress(x, B, fmt=fmt)
    c = codes.cpu().numpy()
    # Blocks whose alpha is not finite in float32 are outside the contract
    # for alpha; codes and s are still compared.
    compare_compress(x, B, c, np.where(np.isfinite(o_a), alpha.cpu().numpy(), o_a),
                     scale.cpu().numpy(), fmt=fmt)
    y = bf16_bits(taco.decompress(to_gpu(o_c), to_gpu(o_a), to_gpu(o_s), block=B, fmt=fmt))
    compare_decompress(y, o_c, o_a, o_s, B, fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_target_energy_only_scales_alpha_and_s(taco, fmt):
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(16, seed=32)
    x = synth.generate(r)
    announce(f"{fmt} tau sweep 16x2560 B=128")
    c1, a1, s1 = [t.cpu().numpy() for t in taco.compress(to_gpu_bf16(x), block=128, fmt=fmt)]
    for tau in (0.125, 1e6):
        ct, at, st = [t.cpu().numpy() for t in taco.compress(to_gpu_bf16(x), block=128,
                                                             target_energy=tau, fmt=fmt)]
        assert np.array_equal(ct, c1)
        np.testing.assert_allclose(at, a1 * tau, rtol=4 * 2.0 ** -23)
        np.testing.assert_allclose(st, s1 * tau, rtol=4 * 2.0 ** -23)


def sample_blocks(M, n, seed):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(64, M)), np.arange(max(0, M - 64), M),
                          rng.integers(0, M, n)])
    return np.unique(idx)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name,B,full", [("gpt2.7b_rowpar_8192x2560", 128, True),
                                         ("grad_8192x8192", 256, True)])
def test_workloads(taco, fmt, name, B, full):
    import torch
    r = synth.WORKLOADS[name]
    announce(f"{fmt} workload {name} B={B}")
    x_bits = synth.generate(r)
    x = to_gpu_bf16(x_bits)
    codes, alpha, scale = taco.compress(x, block=B, fmt=fmt)
    y = taco.decompress(codes, alpha, scale, block=B, fmt=fmt)
    torch.cuda.synchronize()
    M = x_bits.size // B
    idx = np.arange(M) if full else sample_blocks(M, 4096, seed=M)
    tidx = torch.from_numpy(idx).cuda()
    st = compare_compress(x_bits.reshape(M, B)[idx], B, codes.view(M, B)[tidx].cpu().numpy(),
                          alpha[tidx].cpu().numpy(), scale[tidx].cpu().numpy(), fmt=fmt)
    o_c, o_a, o_s = st.pop("oracle")
    ref = synth.bits_to_f32(oracle.decompress(o_c, o_a, o_s, B, fmt=fmt)).astype(np.float64)
    r_rt = rel_rms(synth.bits_to_f32(bf16_bits(y.view(M, B)[tidx])).reshape(-1), ref.reshape(-1))
    assert r_rt <= RECON_RTOL, r_rt
    print(fmt, name, B, st, "roundtrip", r_rt, flush=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B,P", [(64, 0), (128, 1), (256, 3), (512, 8)])
def test_owner_step(taco, fmt, B, P):
    import torch
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(37, 1536)
    announce(f"{fmt} owner step 37x1536 B={B} P={P}")
    own_bits = synth.generate(r, seed=200)
    xs = [synth.generate(r, seed=201 + p) for p in range(P)]
    pay_g, pay_h = [], []
    for v in xs:
        c, a, s = taco.compress(to_gpu_bf16(v), block=B, fmt=fmt)
        pay_g.append((c, a, s))
        pay_h.append((c.cpu().numpy(), a.cpu().numpy(), s.cpu().numpy()))
    codes, alpha, scale = taco.reduce_compress(to_gpu_bf16(own_bits), pay_g, block=B, fmt=fmt)
    torch.cuda.synchronize()
    print(compare_reduce(own_bits, pay_h, B, codes.cpu().numpy(), alpha.cpu().numpy(),
                         scale.cpu().numpy(), fmt=fmt), flush=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [32, 256])
def test_packed_layout_equals_side_buffers(taco, fmt, B):
    import torch
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(8, 3584)
    announce(f"{fmt} packed 8x3584 B={B}")
    x_bits = synth.generate(r, seed=300)
    x = to_gpu_bf16(x_bits)
    c, a, s = taco.compress(x, block=B, fmt=fmt)
    pay = taco.compress_packed(x, block=B, fmt=fmt)
    torch.cuda.synchronize()
    pc, pa, ps = oracle.unpack(pay.cpu().numpy(), B)
    assert np.array_equal(pc, c.cpu().numpy().reshape(-1))
    assert np.array_equal(pa, a.cpu().numpy()) and np.array_equal(ps, s.cpu().numpy())
    y = taco.decompress_packed(pay, x.shape, block=B, fmt=fmt)
    y_side = taco.decompress(c, a, s, block=B, fmt=fmt)
    acc = torch.zeros(x.shape, dtype=torch.float32, device="cuda")
    acc_side = torch.zeros_like(acc)
    taco.decompress_accumulate_packed(pay, acc, block=B, fmt=fmt)
    taco.decompress_accumulate(c, a, s, acc_side, block=B, fmt=fmt)
    out = taco.reduce_compress_packed(x, [pay, pay], block=B, fmt=fmt)
    oc, oa, os_ = taco.reduce_compress(x, [(c, a, s), (c, a, s)], block=B, fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_side.view(torch.int16))
    assert torch.equal(acc, acc_side)
    uc, ua, us = oracle.unpack(out.cpu().numpy(), B)
    assert np.array_equal(uc, oc.cpu().numpy().reshape(-1))
    assert np.array_equal(ua, oa.cpu().numpy()) and np.array_equal(us, os_.cpu().numpy())


def test_format_mismatch_is_the_callers_contract(taco):
    """Formats differ only in the codes: the same input gives the same alpha
    in every format, and s in proportion to 1 / Q_max."""
    import torch
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(4, 1024)
    x = to_gpu_bf16(synth.generate(r, seed=400))
    announce("formats side by side 4x1024 B=128")
    res = {f: taco.compress(x, block=128, fmt=f) for f in ("e4m3", "e5m2", "int8")}
    torch.cuda.synchronize()
    q = taco.QMAX_OF
    for f in FMTS:
        assert torch.equal(res[f][1], res["e4m3"][1])
        ratio = (res[f][2].double() * q[f]) / (res["e4m3"][2].double() * q["e4m3"])
        assert torch.allclose(ratio, torch.ones_like(ratio), rtol=2.0 ** -21)
