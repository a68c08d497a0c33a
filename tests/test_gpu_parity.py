"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Every case prints its name, shape and block before it touches the GPU, so a
failing run names the case it was in.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import (bf16_rel_rms, compare_accumulate, compare_compress, compare_decompress,
                    oracle_accumulate, oracle_decompress, rel_rms, RECON_RTOL)

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


def to_gpu(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def bf16_to_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_compress(taco, x_bits, B, tau=1.0):
    import torch
    x = to_gpu_bf16(x_bits)
    codes, alpha, scale = taco.compress(x, block=B, target_energy=tau)
    torch.cuda.synchronize()
    return codes, alpha, scale


def full_check(taco, x_bits, B, tau=1.0):
    """Compress on the GPU, compare with the oracle, then decompress (and
    accumulate) the oracle's codes on the GPU and compare those too, and
    compare the GPU round trip with the oracle round trip."""
    import torch
    codes, alpha, scale = gpu_compress(taco, x_bits, B, tau)
    st = compare_compress(x_bits, B, codes.cpu().numpy(), alpha.cpu().numpy(),
                          scale.cpu().numpy(), tau)
    o_codes, o_alpha, o_scale = st["oracle"]
    shape = x_bits.shape
    # Decompress kernel alone, on the oracle's payload.
    y = taco.decompress(to_gpu(o_codes.reshape(shape)), to_gpu(o_alpha), to_gpu(o_scale), block=B)
    dst = compare_decompress(bf16_to_bits(y), o_codes, o_alpha, o_scale, B)
    # Accumulate kernel alone: acc starts at a known float32 pattern; every
    # element within the float32 bound of the kernel's arithmetic.
    acc0 = synth.bits_to_f32(x_bits).astype(np.float32).reshape(shape)
    acc = to_gpu(acc0.copy())
    taco.decompress_accumulate(to_gpu(o_codes.reshape(shape)), to_gpu(o_alpha), to_gpu(o_scale),
                               acc, block=B)
    r_acc = compare_accumulate(acc.cpu().numpy(), acc0, [(o_codes, o_alpha, o_scale)],
                               B)["rel_rms"]
    # Round trip: GPU compress + GPU decompress vs the oracle's.
    y2 = taco.decompress(codes, alpha, scale, block=B)
    torch.cuda.synchronize()
    ref = synth.bits_to_f32(oracle.decompress(o_codes, o_alpha, o_scale, B)).astype(np.float64)
    r = rel_rms(synth.bits_to_f32(bf16_to_bits(y2)).reshape(-1), ref.reshape(-1))
    assert r <= RECON_RTOL, f"round trip rel RMS vs oracle {r:.3g}"
    return {**{k: v for k, v in st.items() if k != "oracle"}, "dec_rel": dst["rel_rms"],
            "acc_rel": r_acc, "roundtrip_rel": r}


# ------------------------------------------------------------- codec ------

def test_e4m3_encode_matches_oracle_on_every_float_below_464(taco):
    """Every binary32 value with |v| < 464 (both signs), in chunks."""
    import ctypes
    import torch
    from conftest import build_helper, cpu_threads
    helper = ctypes.CDLL(build_helper("encode_patterns"))
    helper.encode_pattern_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int]
    enc = oracle.encode_function_address()
    limit = int(np.array([464.0], np.float32).view(np.uint32)[0])     # first pattern >= 464
    chunk = 1 << 26
    announce(f"e4m3 encode sweep over {2 * limit} patterns")
    for sign in (0, 1 << 31):
        for lo in range(0, limit, chunk):
            hi = min(lo + chunk, limit)
            pat = torch.arange(lo, hi, dtype=torch.int64, device="cuda").to(torch.int32)
            if sign:
                pat = pat | torch.tensor(-(1 << 31), dtype=torch.int32, device="cuda")
            got = taco.e4m3_encode(pat.view(torch.float32)).cpu().numpy()
            want = np.empty(hi - lo, np.uint8)
            helper.encode_pattern_range(lo | sign, hi | sign, enc,
                                        want.ctypes.data_as(ctypes.c_void_p), cpu_threads())
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (f"pattern {(lo | sign) + int(bad[0]):#010x}: gpu {got[bad[0]]:#x} "
                                   f"oracle {want[bad[0]]:#x} ({bad.size} mismatches)")


def test_e4m3_decode_all_codes(taco):
    import torch
    codes = torch.arange(256, dtype=torch.int32, device="cuda").to(torch.uint8)
    got = taco.e4m3_decode(codes).cpu().numpy().astype(np.float64)
    want = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


# ---------------------------------------------------- block sizes, tails --

@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
def test_all_block_sizes_ragged(taco, B):
    # 37 x 1536 = 56832 elements: for every B the block count is not a
    # multiple of the blocks one wave handles per step.
    r = synth.WORKLOADS["laplace_2048x1024"].with_shape(37, 1536, seed=11)
    announce(f"ragged {r.rows}x{r.cols} B={B}")
    st = full_check(taco, synth.generate(r), B)
    print(st, flush=True)


# Large tensors at B <= 64 run two wave-steps per wave (from 16384 wave-steps
# up).  These shapes give an odd number of wave-steps (16387), so the last
# pair has one wave-step past the end, and a partial last wave-step (3 of 8
# blocks at B = 64, 5 of 16 at B = 32).
PAIRED_SHAPES = [(131091, 64, 64), (262181, 32, 32)]


@pytest.mark.parametrize("tokens,hidden,B", PAIRED_SHAPES)
def test_paired_wave_steps(taco, tokens, hidden, B):
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(tokens, hidden, seed=41)
    announce(f"paired wave-steps {tokens}x{hidden} B={B}")
    st = full_check(taco, synth.generate(r), B)
    print(st, flush=True)


@pytest.mark.parametrize("tokens,hidden,B", [(1, 128, 128), (1, 256, 256), (4, 96, 128),
                                             (3, 32, 32), (5, 512, 512), (7, 64, 64)])
def test_small_and_row_crossing_shapes(taco, tokens, hidden, B):
    r = synth.WORKLOADS["qwen7b_act_16384x3584"].with_shape(tokens, hidden, seed=21)
    announce(f"small {tokens}x{hidden} B={B}")
    full_check(taco, synth.generate(r), B)


def test_empty_tensor_is_a_noop(taco):
    import torch
    announce("empty")
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    codes, alpha, scale = taco.compress(x, block=128)
    assert codes.shape == (0, 1024) and alpha.numel() == 0
    y = taco.decompress(codes, alpha, scale, block=128)
    assert y.shape == (0, 1024)


def test_target_energy_only_scales_alpha_and_s(taco):
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"].with_shape(64, seed=31)
    x = synth.generate(r)
    announce("tau sweep 64x2560 B=128")
    c1, a1, s1 = [t.cpu().numpy() for t in gpu_compress(taco, x, 128, 1.0)]
    for tau in (0.125, 37.5, 1e6):
        full_check(taco, x, 128, tau)
        ct, at, st = [t.cpu().numpy() for t in gpu_compress(taco, x, 128, tau)]
        assert np.array_equal(ct, c1)
        # A few float32 roundings (tau / sigma, then alpha * max * const):
        # at most 4 units in the last place of a float32 (2^-23 relative).
        np.testing.assert_allclose(at, a1 * tau, rtol=4 * 2.0 ** -23)
        np.testing.assert_allclose(st, s1 * tau, rtol=4 * 2.0 ** -23)


# -------------------------------------------------------- special blocks --

def special_blocks(B):
    """Blocks with closed-form results and the kernel's rare branches."""
    from scipy.linalg import hadamard
    H = hadamard(B).astype(np.float64)
    rng = np.random.default_rng(B)
    rows = []
    f = synth.f32_to_bits
    rows.append(np.zeros(B, np.uint16))                                # zero block
    rows.append(np.full(B, 0x8000, np.uint16))                         # negative zeros
    rows.append(f(np.full(B, 0.3)))                                    # constant
    rows.append(f(np.full(B, -7.25)))
    spike = np.zeros(B); spike[B // 3] = -1.5; rows.append(f(spike))   # spike
    rows.append(f(0.5 * H[B // 2 + 1]))                                # Walsh row
    sub = rng.integers(1, 0x7F, B).astype(np.uint16)                   # bf16 subnormals
    sub |= rng.integers(0, 2, B).astype(np.uint16) << 15
    rows.append(sub)
    tiny = rng.standard_normal(B) * 1e-37; rows.append(f(tiny))        # max|R| < 2^-96
    huge = rng.standard_normal(B) * 1e37; rows.append(f(huge))         # sum x^2 overflows
    big = rng.standard_normal(B) * 2.0 ** 70; rows.append(f(big))      # energy >= 2^100
    edge = rng.standard_normal(B) * 3e38 / np.sqrt(B); rows.append(f(edge))
    mixed = rng.laplace(0, 1e-3, B); mixed[::7] = 0.0; mixed[1] = -0.0; rows.append(f(mixed))
    outl = rng.laplace(0, 1e-3, B); outl[5] = 60.0; rows.append(f(outl))   # one dominant value
    pm = np.zeros(B, np.float32); pm[0:B // 2:2] = -0.0; pm[B // 2:] = 0.75
    rows.append(f(pm))                                                 # signed zeros in Z
    ties = np.full(B, 1.0); ties[0] = 448.0 / 17 * 16; rows.append(f(ties))
    # Top of the bf16 range: sum x^2 and B |x| overflow float32.
    rows.append(f(np.full(B, 3.0e38)))
    top = np.clip(rng.standard_normal(B) * 5e37, -2.5e38, 2.5e38); rows.append(f(top))
    return np.stack(rows)


@pytest.mark.parametrize("B", [32, 128, 256, 512])
def test_special_blocks(taco, B):
    x = special_blocks(B)
    announce(f"special blocks B={B} ({x.shape[0]} blocks)")
    codes, alpha, scale = gpu_compress(taco, x, B)
    c, a, s = codes.cpu().numpy(), alpha.cpu().numpy(), scale.cpu().numpy()
    o_c, o_a, o_s = oracle.compress(x, B)
    assert np.array_equal(c, o_c), np.argwhere(c != o_c)[:10]
    finite = np.isfinite(o_a)
    np.testing.assert_allclose(a[finite], o_a[finite], rtol=1e-6)
    np.testing.assert_allclose(s, o_s, rtol=1e-6)
    y = bf16_to_bits(taco.decompress(codes, alpha, scale, block=B))
    ref = synth.bits_to_f32(oracle.decompress(o_c, o_a, o_s, B)).astype(np.float64)
    yf = synth.bits_to_f32(y).astype(np.float64)
    for k in range(x.shape[0]):
        assert rel_rms(yf[k], ref[k]) <= RECON_RTOL, k
    compare_decompress(y, o_c, o_a, o_s, B)


# ------------------------------------------------------ the five workloads --
# Every workload is compared in full (every block, every element), at the
# block size and in the launch configuration the benchmark times.

def workload_check(taco, name, B, seed=None):
    """Compress and decompress a whole workload on the GPU.  Codes, alpha and
    s of every block against the oracle; the decompress kernel on the
    oracle's payload, every element; the GPU round trip against the
    oracle's round trip (relative RMS)."""
    import torch
    r = synth.WORKLOADS[name]
    announce(f"workload {name} B={B} seed={seed if seed is not None else r.seed} (full)")
    x_bits = synth.generate(r, seed=seed)
    shape = x_bits.shape
    x = to_gpu_bf16(x_bits)
    codes, alpha, scale = taco.compress(x, block=B)
    y = taco.decompress(codes, alpha, scale, block=B)
    torch.cuda.synchronize()
    st = compare_compress(x_bits, B, codes.cpu().numpy(), alpha.cpu().numpy(),
                          scale.cpu().numpy())
    o_c, o_a, o_s = st.pop("oracle")
    y_o = taco.decompress(to_gpu(o_c.reshape(shape)), to_gpu(o_a), to_gpu(o_s), block=B)
    st["decompress_rel"] = compare_decompress(bf16_to_bits(y_o), o_c, o_a, o_s, B)["rel_rms"]
    st["roundtrip_rel"] = bf16_rel_rms(bf16_to_bits(y), oracle_decompress(o_c, o_a, o_s, B))
    assert st["roundtrip_rel"] <= RECON_RTOL, st
    print(name, B, st, flush=True)
    return st


def test_workload_laplace_full(taco):
    workload_check(taco, "laplace_2048x1024", 128)


def test_workload_gpt27b_rowparallel_full(taco):
    workload_check(taco, "gpt2.7b_rowpar_8192x2560", 128)


@pytest.mark.parametrize("B", [128, 256])
def test_workload_qwen7b_activation_full(taco, B):
    workload_check(taco, "qwen7b_act_16384x3584", B)


def test_workload_gradient_full(taco):
    workload_check(taco, "grad_8192x8192", 256)


@pytest.fixture(scope="module")
def gpt175b_state():
    """Accumulators of the four-payload workload, shared by its tests (one
    test per payload keeps each under a minute): the GPU pipeline's (its own
    codes), the GPU accumulate kernel's on the oracle's payloads, and the
    oracle's."""
    return {"done": []}


@pytest.mark.parametrize("p", range(4))
def test_workload_gpt175b_payload_full(taco, gpt175b_state, p):
    """Largest workload (four independently seeded payloads compressed and
    summed into one float32 accumulator, as the benchmark times it), payload
    p: every block against the oracle; then the accumulate kernel on the
    oracle's payload, every element within its float32 bound on the input it
    was given; the GPU pipeline accumulates the GPU's own payload."""
    import torch
    name, B = "gpt175b_hidden_32768x12288", 256
    r = synth.WORKLOADS[name]
    st8 = gpt175b_state
    assert st8["done"] == list(range(p)), "payloads run in order"
    if p == 0:
        st8["acc"] = torch.zeros((r.rows, r.cols), dtype=torch.float32, device="cuda")
        st8["acc_k"] = torch.zeros((r.rows, r.cols), dtype=torch.float32, device="cuda")
        st8["ref"] = np.zeros(r.numel, np.float32)
    seed = synth.ACCUMULATE_SEEDS[p]
    announce(f"{name} payload {p} seed={seed} (full)")
    x_bits = synth.generate(r, seed=seed)
    x = to_gpu_bf16(x_bits)
    codes, alpha, scale = taco.compress(x, block=B)
    taco.decompress_accumulate(codes, alpha, scale, st8["acc"], block=B)
    torch.cuda.synchronize()
    st = compare_compress(x_bits, B, codes.cpu().numpy(), alpha.cpu().numpy(),
                          scale.cpu().numpy())
    del x, codes, alpha, scale, x_bits
    o_c, o_a, o_s = st.pop("oracle")
    print(name, B, f"payload {p}", st, flush=True)
    before = st8["acc_k"].cpu().numpy().reshape(-1)
    taco.decompress_accumulate(to_gpu(o_c.reshape(r.rows, r.cols)), to_gpu(o_a), to_gpu(o_s),
                               st8["acc_k"], block=B)
    torch.cuda.synchronize()
    ka = compare_accumulate(st8["acc_k"].cpu().numpy(), before, [(o_c, o_a, o_s)], B)
    print("accumulate kernel step vs oracle", ka, flush=True)
    # Beside the worst-case bound, the tighter one that holds in practice.
    assert ka["max_err_over_block_magnitude"] <= 2.0 ** -20, ka
    oracle_accumulate(o_c, o_a, o_s, B, st8["ref"])
    st8["done"].append(p)


def test_workload_gpt175b_accumulators(taco, gpt175b_state):
    """After the four payloads: the GPU pipeline's accumulator and the
    kernel's (on the oracle's payloads) against the oracle's accumulator."""
    st8 = gpt175b_state
    assert st8["done"] == [0, 1, 2, 3]
    announce("gpt175b accumulators vs the oracle's (full)")
    ref = st8["ref"]
    r_k = rel_rms(st8["acc_k"].cpu().numpy().reshape(-1), ref)
    r_acc = rel_rms(st8["acc"].cpu().numpy().reshape(-1), ref)
    print("accumulator rel RMS vs oracle: kernel", r_k, "pipeline", r_acc, flush=True)
    assert r_k <= 1e-6
    assert r_acc <= RECON_RTOL
    st8.clear()


# ------------------------------------------------------ launch behaviour --

def test_deterministic_and_stream_ordered(taco):
    import torch
    r = synth.WORKLOADS["grad_8192x8192"].with_shape(512)
    x_bits = synth.generate(r)
    announce("determinism + side stream")
    x = to_gpu_bf16(x_bits)
    c1, a1, s1 = taco.compress(x, block=256)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c2, a2, s2 = taco.compress(x, block=256)
        y2 = taco.decompress(c2, a2, s2, block=256)
    torch.cuda.current_stream().wait_stream(side)
    y1 = taco.decompress(c1, a1, s1, block=256)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(a1, a2) and torch.equal(s1, s2)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
