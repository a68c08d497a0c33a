"""Properties that hold at any size, checked on every element of full-size
workloads (no oracle call needed).  Scaling X by 2^k changes only exponents:
R = H X, max|R| and the block energy scale exactly, so the codes of
Q R / max|R| and s = alpha max|R| / (sqrt(B) Q) are bit-identical, alpha
scales by exactly 2^-k, and the reconstruction scales by exactly 2^k
([TACO] Eq. 6-13; the same invariance pins the oracle).  The target energy
tau scales alpha and s and leaves the codes alone ([TACO] Eq. 7).  Energies
stay far above the epsilon of Eq. 6 and away from the rescaling branches."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def taco():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gradients_taco_compress_amd as taco
    return taco


def to_gpu_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def scaled_bits(bits, k):
    """bf16 bit patterns times 2^k (exponent shift; inputs stay normal)."""
    b = np.ascontiguousarray(bits).astype(np.int32)
    exp = (b >> 7) & 0xFF
    nz = exp != 0
    assert np.all((exp[nz] + k > 0) & (exp[nz] + k < 255)), "scaled value leaves the normal range"
    assert np.all(exp[~nz] == 0) and np.all((b[~nz] & 0x7F) == 0), "subnormal input"
    out = np.where(nz, b + (k << 7), b)
    return out.astype(np.uint16).reshape(np.shape(bits))


CASES = [("gpt2.7b_rowpar_8192x2560", None, 128, (-4, 5)),
         ("grad_8192x8192", None, 256, (6,)),
         ("laplace_2048x1024", (131091, 64), 64, (-3,)),      # paired wave-steps
         ("laplace_2048x1024", (262181, 32), 32, (3,)),       # paired wave-steps
         ("qwen7b_act_16384x3584", (2048, 3584), 512, (-2, 7))]


@pytest.mark.parametrize("name,shape,B,ks", CASES)
def test_power_of_two_scaling(taco, name, shape, B, ks):
    import torch
    r = synth.WORKLOADS[name]
    if shape is not None:
        r = r.with_shape(*shape)
    x = synth.generate(r)
    print(f"[case] 2^k scaling {r.rows}x{r.cols} B={B} k={ks}", flush=True)
    c0, a0, s0 = taco.compress(to_gpu_bf16(x), block=B)
    y0 = taco.decompress(c0, a0, s0, block=B)
    torch.cuda.synchronize()
    c0, a0, s0 = c0.cpu().numpy(), a0.cpu().numpy(), s0.cpu().numpy()
    y0 = y0.view(torch.int16).cpu().numpy().view(np.uint16)
    for k in ks:
        ck, ak, sk = taco.compress(to_gpu_bf16(scaled_bits(x, k)), block=B)
        yk = taco.decompress(ck, ak, sk, block=B)
        torch.cuda.synchronize()
        assert np.array_equal(ck.cpu().numpy(), c0), f"codes differ for k={k}"
        assert np.array_equal(sk.cpu().numpy(), s0), f"s differs for k={k}"
        assert np.array_equal(ak.cpu().numpy(), np.ldexp(a0, -k)), f"alpha not scaled for k={k}"
        yk = yk.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(yk, scaled_bits(y0, k)), f"reconstruction not scaled for k={k}"


def test_target_energy_at_full_size(taco):
    import torch
    r = synth.WORKLOADS["gpt2.7b_rowpar_8192x2560"]
    x = to_gpu_bf16(synth.generate(r))
    print("[case] tau at full size 8192x2560 B=128", flush=True)
    c1, a1, s1 = [t.cpu().numpy() for t in taco.compress(x, block=128)]
    for tau in (0.25, 37.5):
        ct, at, st = taco.compress(x, block=128, target_energy=tau)
        torch.cuda.synchronize()
        assert np.array_equal(ct.cpu().numpy(), c1)
        np.testing.assert_allclose(at.cpu().numpy(), a1 * tau, rtol=4 * 2.0 ** -23)
        np.testing.assert_allclose(st.cpu().numpy(), s1 * tau, rtol=4 * 2.0 ** -23)


SPLIT_CASES = [("gpt2.7b_rowpar_8192x2560", None, 128),
               ("laplace_2048x1024", (131091, 64), 64),       # whole call paired, pieces not
               ("qwen7b_act_16384x3584", (2048, 3584), 512)]


@pytest.mark.parametrize("name,shape,B", SPLIT_CASES)
def test_split_at_block_boundaries(taco, name, shape, B):
    """Blocks are independent: compressing (and decompressing, and
    accumulating) a tensor in
    pieces cut at arbitrary block boundaries, each piece its own call, gives
    exactly the bytes of one call (the property sharding relies on).  The
    cuts fall inside wave-steps, so every piece ends on a partial one."""
    import torch
    r = synth.WORKLOADS[name]
    if shape is not None:
        r = r.with_shape(*shape)
    n = r.rows * r.cols
    m = n // B
    print(f"[case] split calls {r.rows}x{r.cols} B={B}", flush=True)
    x = to_gpu_bf16(synth.generate(r)).reshape(-1)
    c1, a1, s1 = taco.compress(x, block=B)
    y1 = taco.decompress(c1, a1, s1, block=B)
    cuts = sorted({0, 1, 7, 11, 3 * m // 7 + 5, m - 3, m})
    c2 = torch.empty_like(c1)
    a2 = torch.empty_like(a1)
    s2 = torch.empty_like(s1)
    y2 = torch.empty_like(y1)
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        taco.compress(x[lo * B:hi * B], block=B, codes=c2[lo * B:hi * B], alpha=a2[lo:hi],
                      scale=s2[lo:hi])
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        taco.decompress(c2[lo * B:hi * B], a2[lo:hi], s2[lo:hi], block=B, out=y2[lo * B:hi * B])
    acc1 = torch.full((n,), 0.5, dtype=torch.float32, device="cuda")
    acc2 = acc1.clone()
    taco.decompress_accumulate(c1, a1, s1, acc1, block=B)
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        taco.decompress_accumulate(c2[lo * B:hi * B], a2[lo:hi], s2[lo:hi], acc2[lo * B:hi * B],
                                   block=B)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(a1, a2) and torch.equal(s1, s2)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(acc1, acc2)
