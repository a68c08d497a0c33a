"""The entry points inside a HIP graph, the way bench.py times them.

One graph captures compress, decompress, accumulate, the multi-payload
accumulate, the owner step, the interleaved pair and a fidelity round trip
(accumulators are reset by a copy inside the graph).  It is replayed several
times with eager launches and synchronisations in between, and every replay
must give exactly what the eager calls give (the fidelity sums, which the
kernels add with atomics in an unspecified order, to 1e-12 relative).

Every case prints its name before it touches the GPU.
"""
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


def announce(msg):
    print(f"[case] {msg}", flush=True)


def to_gpu_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
def test_graph_replays_equal_eager_calls(taco, fmt):
    import torch
    B, rows, cols = 128, 96, 1024
    announce(f"graph replays vs eager, {rows}x{cols}, B={B}, {fmt}")
    base = synth.WORKLOADS["laplace_2048x1024"]
    xs = [to_gpu_bf16(synth.generate(base.with_shape(rows), seed=50 + i)) for i in range(4)]
    x, own, pays_x = xs[0], xs[1], xs[1:]
    acc0 = torch.randn(rows, cols, device="cuda", dtype=torch.float32) * 0.01
    n, m = rows * cols, rows * cols // B

    # Payloads (inputs of the receive calls), made once, eagerly.
    pays = [taco.compress(p, block=B, fmt=fmt) for p in pays_x]
    packed_in = taco.compress_packed(x, block=B, fmt=fmt)

    def run(out):
        taco.compress(x, block=B, fmt=fmt, codes=out["codes"], alpha=out["alpha"],
                      scale=out["scale"])
        taco.decompress(out["codes"], out["alpha"], out["scale"], block=B, fmt=fmt, out=out["y"])
        out["acc"].copy_(acc0)
        taco.decompress_accumulate(*pays[0], out["acc"], block=B, fmt=fmt)
        out["accn"].copy_(acc0)
        taco.decompress_accumulate_n(pays, out["accn"], block=B, fmt=fmt)
        taco.reduce_compress(own, pays[1:], block=B, fmt=fmt, codes=out["rc_codes"],
                             alpha=out["rc_alpha"], scale=out["rc_scale"])
        taco.compress_packed(x, block=B, fmt=fmt, payload=out["packed"])
        taco.decompress_packed(packed_in, x.shape, block=B, fmt=fmt, out=out["y_packed"])
        taco.roundtrip(x, block=B, variant="taco", fmt=fmt, sums=out["sums"], out=out["y_rt"])

    def buffers():
        return {
            "codes": torch.empty(rows, cols, dtype=torch.uint8, device="cuda"),
            "alpha": torch.empty(m, device="cuda"), "scale": torch.empty(m, device="cuda"),
            "y": torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda"),
            "acc": torch.empty(rows, cols, device="cuda"),
            "accn": torch.empty(rows, cols, device="cuda"),
            "rc_codes": torch.empty(rows, cols, dtype=torch.uint8, device="cuda"),
            "rc_alpha": torch.empty(m, device="cuda"), "rc_scale": torch.empty(m, device="cuda"),
            "packed": torch.empty(taco.taco_packed_bytes(rows, cols, B), dtype=torch.uint8,
                                  device="cuda"),
            "y_packed": torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda"),
            "y_rt": torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda"),
            "sums": torch.empty(taco.FIDELITY_SUMS_BYTES, dtype=torch.uint8, device="cuda"),
        }

    eager = buffers()
    run(eager)
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in eager.items()}
    want_metrics = taco.fidelity_metrics(want["sums"], n)

    graphed = buffers()
    run(graphed)                                   # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graphed)
    other = buffers()
    for rep in range(4):
        announce(f"replay {rep}")
        for v in graphed.values():                 # stale contents must not survive
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        run(other)                                 # eager work between replays
        torch.cuda.synchronize()
        for k in want:
            if k == "sums":
                continue
            assert torch.equal(graphed[k], want[k]), f"replay {rep}: {k} differs from eager"
        got = taco.fidelity_metrics(graphed["sums"], n)
        for key in ("rel_l2", "cos", "max_err", "mse"):
            assert got[key] == pytest.approx(want_metrics[key], rel=1e-12, abs=0.0), (rep, key)
        for k in want:
            if k != "sums":
                assert torch.equal(other[k], want[k]), f"eager call after replay {rep}: {k}"


def test_noalloc_round_trip_in_a_graph(taco):
    """taco_roundtrip_noalloc captured in a graph (its working sums live in
    the library's per-GPU array, cleared by a kernel, so the graph holds no
    memset and no allocation): every replay equals the eager call, with eager
    calls on another tensor, sharing the same array, in between."""
    import struct
    import torch
    B, rows, cols = 256, 64, 2048
    announce(f"noalloc round trip in a graph, {rows}x{cols}, B={B}")
    base = synth.WORKLOADS["grad_8192x8192"]
    x = to_gpu_bf16(synth.generate(base.with_shape(rows, cols), seed=70))
    x2 = to_gpu_bf16(synth.generate(base.with_shape(rows // 2, cols), seed=71))
    f, v = taco.FORMATS["int8"], taco.VARIANTS["tensor"]

    def call(xt, y, t):
        r, c = xt.shape
        st = taco.taco_roundtrip_noalloc(xt.data_ptr(), r, c, B, 1.0, f, v, y.data_ptr(),
                                         t.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0, taco.taco_status_string(st)

    def totals(t):
        return struct.unpack("<4d2f", bytes(t.cpu().numpy().tobytes()))

    def out_for(xt):
        return (torch.empty_like(xt),
                torch.empty(taco.FIDELITY_TOTALS_BYTES, dtype=torch.uint8, device="cuda"))

    y_ref, t_ref = out_for(x)
    y2_ref, t2_ref = out_for(x2)
    call(x, y_ref, t_ref)                 # the first call (outside capture) looks up the array
    call(x2, y2_ref, t2_ref)
    torch.cuda.synchronize()
    want, want2 = totals(t_ref), totals(t2_ref)

    y_g, t_g = out_for(x)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(x, y_g, t_g)
    y2, t2 = out_for(x2)
    for rep in range(4):
        announce(f"noalloc replay {rep}")
        y_g.zero_()
        t_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        call(x2, y2, t2)                  # eager, same stream, same working array
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_ref.view(torch.int16)), rep
        got = totals(t_g)
        for a, b in zip(got[:4], want[:4]):
            assert a == pytest.approx(b, rel=1e-12, abs=0.0), rep
        assert got[4:] == want[4:], rep
        assert torch.equal(y2.view(torch.int16), y2_ref.view(torch.int16)), rep
        got2 = totals(t2)
        for a, b in zip(got2[:4], want2[:4]):
            assert a == pytest.approx(b, rel=1e-12, abs=0.0), rep
        assert got2[4:] == want2[4:], rep
