"""The measurement kernels of libtaco_probe on the GPU: the plain streams
read and write exactly the bytes they are timed for (so the floors in the
bench line are honest), and the empty kernel runs on any grid.

Every case prints its name before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gradients_taco_compress_amd.probe as probe
    return probe


@pytest.mark.parametrize("mix", ["compress", "decompress", "accumulate", "copy"])
def test_stream_writes_the_xor_of_what_it_reads(probe, mix):
    """Wavefront w, lane l: its KiB j of dst holds, per 32-bit word, the XOR
    of the words at the same lane offset in its `loads` KiB of src, plus j.
    A sentinel after dst must survive (nothing written past the end)."""
    import torch
    ld, st = probe.MIXES[mix]
    waves = 37                                   # not a multiple of 4: a partial work-group
    print(f"[case] probe stream {mix} ({ld}, {st}) waves={waves}", flush=True)
    rng = np.random.default_rng(ld * 10 + st)
    src_h = rng.integers(0, 2 ** 32, size=waves * ld * 256, dtype=np.uint32)
    src = torch.from_numpy(src_h.view(np.int32)).cuda()
    dst = torch.full((waves * st * 256 + 256,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    probe.stream(mix, src, dst, waves)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32)
    x = src_h.reshape(waves, ld, 256)
    acc = np.bitwise_xor.reduce(x, axis=1)                   # [waves, 256 words]
    want = np.stack([(acc + np.uint32(j)) for j in range(st)], axis=1).reshape(-1)
    assert np.array_equal(got[:waves * st * 256], want)
    assert np.all(got[waves * st * 256:] == 0x5A5A5A5A)


def test_stream_with_arithmetic_writes_every_byte(probe):
    import torch
    waves = 64
    print(f"[case] probe stream with VALU load, waves={waves}", flush=True)
    src = torch.ones(waves * 2 * 512, dtype=torch.bfloat16, device="cuda")
    dst = torch.full((waves * 1024 + 64,), 0x77, dtype=torch.uint8, device="cuda")
    probe.stream("compress", src, dst, waves, valu=276)
    torch.cuda.synchronize()
    d = dst.cpu().numpy()
    words = d[:waves * 1024].view(np.uint32)
    assert not np.any(words == 0x77777777)        # every word of the output rewritten
    assert np.all(d[waves * 1024:] == 0x77)


@pytest.mark.parametrize("groups", [1, 512, 49152])
def test_empty_kernel(probe, groups):
    import torch
    print(f"[case] probe empty groups={groups}", flush=True)
    probe.empty(groups)
    torch.cuda.synchronize()


def test_bad_arguments_are_refused(probe):
    import torch
    print("[case] probe argument checks", flush=True)
    a = torch.empty(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        probe.stream("compress", a, a, 100)                   # buffers too small
    assert probe.taco_probe_stream(3, 1, 0, a.data_ptr(), a.data_ptr() + 2048, 1, 0) == 1
    assert probe.taco_probe_empty(0, 0) == 1
