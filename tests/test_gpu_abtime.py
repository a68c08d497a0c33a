"""The A/B timer on the GPU: the same build twice gives identical outputs and
positive times for every operation (a small run)."""
import os

import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gradients_taco_compress_amd", "libtaco.so")


def test_same_build_twice():
    import torch
    from gradients_taco_compress_amd import abtime
    print("[case] abtime laplace_2048x1024 B=128, the default build twice", flush=True)
    res = abtime.compare([LIB, LIB], "laplace_2048x1024", 128, repeats=2,
                         rotate_bytes=16 << 20, launches=8)
    torch.cuda.empty_cache()
    assert res["identical_outputs"] is True
    assert res["sets"] == 8 and res["launches_per_graph"] == 8
    assert sorted(res["builds"]) == ["0:libtaco.so", "1:libtaco.so"]
    for build in res["builds"].values():
        assert sorted(build) == sorted(abtime.OPS)
        for op in build.values():
            assert op["us"] > 0 and op["GBps"] > 0
