"""Tensors past 2^31 elements (the largest sizes the 64-bit element indexing
has to carry), on the GPU through the C ABI: sampled blocks around the 2^31
boundary and at the end against the oracle.  Inputs are seeded normals drawn
on the GPU (torch's generator), rounded to bf16."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import compare_compress, rel_rms, RECON_RTOL

pytestmark = pytest.mark.gpu

TOKENS, HIDDEN, B = 131073, 16384, 256          # N = 2^31 + 16384 elements


@pytest.fixture(scope="module")
def taco():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gradients_taco_compress_amd as taco
    return taco


def sample_blocks(M):
    """Blocks at the start, just before and after element 2^31, and at the end."""
    edge = (1 << 31) // B
    idx = np.concatenate([np.arange(0, 8), np.arange(edge - 16, edge + 16), np.arange(M - 16, M)])
    return np.unique(idx)


def test_past_two_to_the_31(taco):
    import torch
    n = TOKENS * HIDDEN
    assert n > (1 << 31)
    M = n // B
    print(f"[case] large {TOKENS}x{HIDDEN} B={B} (N = {n})", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    x = (torch.randn((TOKENS, HIDDEN), generator=g, device="cuda", dtype=torch.float32) * 0.02)
    x = x.to(torch.bfloat16)
    idx = sample_blocks(M)
    tidx = torch.from_numpy(idx).cuda()
    xb = x.view(M, B)[tidx].view(torch.int16).cpu().numpy().view(np.uint16)

    codes, alpha, scale = taco.compress(x, block=B)
    torch.cuda.synchronize()
    st = compare_compress(xb, B, codes.view(M, B)[tidx].cpu().numpy(), alpha[tidx].cpu().numpy(),
                          scale[tidx].cpu().numpy())
    o_c, o_a, o_s = st.pop("oracle")
    print("compress", st, flush=True)

    y = taco.decompress(codes, alpha, scale, block=B)
    torch.cuda.synchronize()
    ref = synth.bits_to_f32(oracle.decompress(o_c, o_a, o_s, B)).astype(np.float64).reshape(-1)
    got = synth.bits_to_f32(y.view(M, B)[tidx].view(torch.int16).cpu().numpy().view(np.uint16))
    r = rel_rms(got.reshape(-1), ref)
    assert r <= RECON_RTOL, r
    del y

    # Interleaved layout: the same codes and scalars, record by record.
    pay = taco.compress_packed(x, block=B)
    torch.cuda.synchronize()
    rec = pay.view(M, B + 8)[tidx].cpu().numpy()
    pc, pa, ps = oracle.unpack(rec, B)
    assert np.array_equal(pc, codes.view(M, B)[tidx].cpu().numpy().reshape(-1))
    assert np.array_equal(pa, alpha[tidx].cpu().numpy())
    assert np.array_equal(ps, scale[tidx].cpu().numpy())
    del pay, x

    acc = torch.zeros((TOKENS, HIDDEN), dtype=torch.float32, device="cuda")
    taco.decompress_accumulate(codes, alpha, scale, acc, block=B)
    taco.decompress_accumulate(codes, alpha, scale, acc, block=B)
    torch.cuda.synchronize()
    want = oracle.decompress_accumulate(o_c, o_a, o_s, B, np.zeros(idx.size * B, np.float32))
    want = oracle.decompress_accumulate(o_c, o_a, o_s, B, want)
    r = rel_rms(acc.view(M, B)[tidx].cpu().numpy().reshape(-1), want)
    assert r <= 1e-6, r
