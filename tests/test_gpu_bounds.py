"""No entry point writes past its outputs.

Every writing entry point runs on tensors whose last wave-step holds an odd
number of blocks (so the staged stores end in a short piece: an interleaved
record run is then not a multiple of 16 bytes), for every block size, with
each output placed at the front of a larger buffer whose tail holds a known
pattern; the tail must be unchanged afterwards, and the results must equal
those written into exact-size buffers.

Every case prints its name before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of guard after each output


@pytest.fixture(scope="module")
def taco():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gradients_taco_compress_amd as taco
    return taco


def announce(msg):
    print(f"[case] {msg}", flush=True)


def guarded(n, dtype, fill):
    """(view of n elements, whole buffer, the tail's expected contents)."""
    import torch
    extra = GUARD // torch.empty(0, dtype=dtype).element_size()
    buf = torch.full((n + extra,), fill, dtype=dtype, device="cuda")
    return buf[:n], buf, buf[n:].clone()


def assert_tail(buf, n, tail, what):
    import torch
    torch.cuda.synchronize()
    assert torch.equal(buf[n:], tail), f"{what}: bytes past the output were written"


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512])
def test_outputs_are_not_overrun(taco, B):
    import torch
    bpw = 16 if B == 32 else 8                     # blocks per wave-step
    nblocks = 3 * bpw + 3                          # last wave-step: 3 blocks
    cols = B * nblocks
    base = synth.WORKLOADS["laplace_2048x1024"]
    xs = [torch.from_numpy(synth.generate(base.with_shape(1, cols), seed=70 + i).view(np.int16))
          .cuda().view(torch.bfloat16) for i in range(3)]
    x = xs[0]
    n, m = cols, nblocks
    nb = taco.taco_packed_bytes(1, cols, B)
    announce(f"guarded outputs 1x{cols} B={B} ({nblocks} blocks)")

    # compress, side buffers
    c, cb, ct = guarded(n, torch.uint8, 0xAB)
    a, ab, at = guarded(m, torch.float32, 12345.0)
    s, sb, stl = guarded(m, torch.float32, 12345.0)
    taco.compress(x, block=B, codes=c, alpha=a, scale=s)
    assert_tail(cb, n, ct, "compress codes")
    assert_tail(ab, m, at, "compress alpha")
    assert_tail(sb, m, stl, "compress scale")
    ref = taco.compress(x, block=B)
    assert torch.equal(c, ref[0].view(-1)) and torch.equal(a, ref[1]) and torch.equal(s, ref[2])

    # compress, interleaved records
    pk, pkb, pkt = guarded(nb, torch.uint8, 0xCD)
    taco.compress_packed(x, block=B, payload=pk)
    assert_tail(pkb, nb, pkt, "compress_packed")
    assert torch.equal(pk, taco.compress_packed(x, block=B))

    # decompress and accumulate, both layouts
    y, yb, yt = guarded(n, torch.bfloat16, 3.0)
    taco.decompress(c, a, s, block=B, out=y.view(1, n))
    assert_tail(yb, n, yt, "decompress")
    y2, y2b, y2t = guarded(n, torch.bfloat16, 3.0)
    taco.decompress_packed(pk, (1, n), block=B, out=y2.view(1, n))
    assert_tail(y2b, n, y2t, "decompress_packed")
    assert torch.equal(y, y2)
    acc, accb, acct = guarded(n, torch.float32, 7.0)
    acc.zero_()
    taco.decompress_accumulate(c, a, s, acc, block=B)
    assert_tail(accb, n, acct, "decompress_accumulate")
    acc2, acc2b, acc2t = guarded(n, torch.float32, 7.0)
    acc2.zero_()
    taco.decompress_accumulate_packed(pk, acc2, block=B)
    assert_tail(acc2b, n, acc2t, "decompress_accumulate_packed")
    assert torch.equal(acc, acc2)

    # several payloads at once, both layouts
    pays = [taco.compress(v, block=B) for v in xs[1:]]
    ppays = [taco.compress_packed(v, block=B) for v in xs[1:]]
    accn, accnb, accnt = guarded(n, torch.float32, 7.0)
    accn.zero_()
    taco.decompress_accumulate_n(pays, accn.view(1, n), block=B)
    assert_tail(accnb, n, accnt, "decompress_accumulate_n")
    accp, accpb, accpt = guarded(n, torch.float32, 7.0)
    accp.zero_()
    taco.decompress_accumulate_n_packed(ppays, accp.view(1, n), block=B)
    assert_tail(accpb, n, accpt, "decompress_accumulate_n_packed")
    assert torch.equal(accn, accp)

    # owner step, both layouts
    rc, rcb, rct = guarded(n, torch.uint8, 0xAB)
    ra, rab, rat = guarded(m, torch.float32, 12345.0)
    rs, rsb, rst = guarded(m, torch.float32, 12345.0)
    taco.reduce_compress(x, pays, block=B, codes=rc, alpha=ra, scale=rs)
    assert_tail(rcb, n, rct, "reduce_compress codes")
    assert_tail(rab, m, rat, "reduce_compress alpha")
    assert_tail(rsb, m, rst, "reduce_compress scale")
    rp, rpb, rpt = guarded(nb, torch.uint8, 0xCD)
    taco.reduce_compress_packed(x, ppays, block=B, out=rp)
    assert_tail(rpb, nb, rpt, "reduce_compress_packed")
    assert torch.equal(rp, taco.reduce_compress_packed(x, ppays, block=B))

    # fidelity round trip with its output
    yr, yrb, yrt = guarded(n, torch.bfloat16, 3.0)
    taco.roundtrip(x, block=B, out=yr.view(1, n))
    assert_tail(yrb, n, yrt, "roundtrip")
    assert torch.equal(yr, y)


def test_binding_refuses_short_outputs(taco):
    import torch
    announce("short outputs refused")
    x = torch.zeros(4, 512, dtype=torch.bfloat16, device="cuda")
    pk = taco.compress_packed(x, block=128)
    with pytest.raises(ValueError):
        taco.decompress_packed(pk, (4, 512), block=128,
                               out=torch.empty(4, 256, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        taco.reduce_compress_packed(x, [pk], block=128,
                                    out=torch.empty(pk.numel() - 8, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        taco.encode(torch.zeros(64, device="cuda"), out=torch.empty(32, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        taco.decode(torch.zeros(64, dtype=torch.uint8, device="cuda"),
                    out=torch.empty(32, device="cuda"))


@pytest.mark.parametrize("B", [128, 256])
def test_non_finite_inputs_stay_in_bounds(taco, B):
    """Non-finite inputs give unspecified codes and scalars, but every call
    still returns TACO_OK and writes only its outputs."""
    import torch
    bpw = 8
    nblocks = 2 * bpw + 5
    n = B * nblocks
    announce(f"non-finite inputs 1x{n} B={B}")
    base = synth.WORKLOADS["laplace_2048x1024"]
    x = torch.from_numpy(synth.generate(base.with_shape(1, n), seed=90).view(np.int16)).cuda()
    x = x.view(torch.bfloat16).clone()
    x[0, 3] = float("nan")
    x[0, B + 7] = float("inf")
    x[0, 5 * B] = float("-inf")
    x[0, 6 * B:7 * B] = float("nan")                 # a whole NaN block
    m = nblocks
    nb = taco.taco_packed_bytes(1, n, B)
    c, cb, ct = guarded(n, torch.uint8, 0xAB)
    a, ab, at = guarded(m, torch.float32, 12345.0)
    s, sb, stl = guarded(m, torch.float32, 12345.0)
    taco.compress(x, block=B, codes=c, alpha=a, scale=s)
    for buf, k, tail, what in ((cb, n, ct, "codes"), (ab, m, at, "alpha"), (sb, m, stl, "scale")):
        assert_tail(buf, k, tail, what)
    pk, pkb, pkt = guarded(nb, torch.uint8, 0xCD)
    taco.compress_packed(x, block=B, payload=pk)
    assert_tail(pkb, nb, pkt, "compress_packed")
    y, yb, yt = guarded(n, torch.bfloat16, 3.0)
    taco.decompress(c, a, s, block=B, out=y.view(1, n))
    assert_tail(yb, n, yt, "decompress")
    acc, accb, acct = guarded(n, torch.float32, 7.0)
    acc.zero_()
    taco.decompress_accumulate_n([(c, a, s), (c, a, s)], acc.view(1, n), block=B)
    assert_tail(accb, n, acct, "decompress_accumulate_n")
    rp, rpb, rpt = guarded(nb, torch.uint8, 0xCD)
    taco.reduce_compress_packed(x, [pk], block=B, out=rp)
    assert_tail(rpb, nb, rpt, "reduce_compress_packed")
    yr, yrb, yrt = guarded(n, torch.bfloat16, 3.0)
    taco.roundtrip(x, block=B, variant="tensor", out=yr.view(1, n))
    assert_tail(yrb, n, yrt, "roundtrip")
    # Blocks without a non-finite value are unaffected by their neighbours.
    clean = x.clone()
    clean[0, :8 * B] = 0.0
    cc, ca, cs = taco.compress(clean, block=B)
    fin = torch.isfinite(x.view(nblocks, B).float()).all(dim=1)
    fin[:8] = False
    assert torch.equal(cc.view(nblocks, B)[fin], c.view(nblocks, B)[fin])
