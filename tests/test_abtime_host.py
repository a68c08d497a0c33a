"""The A/B timing module's host side (no GPU): loading a build, the bytes it
counts per launch, and its argument checks."""
import ctypes
import os

import pytest

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gradients_taco_compress_amd", "libtaco.so")


def test_load_sets_the_argument_types():
    from gradients_taco_compress_amd import abtime
    if not os.path.exists(LIB):
        pytest.fail("libtaco.so is not built; run __graft_entry__.build()")
    lib = abtime.load(LIB)
    assert len(lib.taco_compress.argtypes) == 9
    assert len(lib.taco_decompress.argtypes) == 8
    assert len(lib.taco_decompress_accumulate.argtypes) == 8
    assert lib.taco_compress.restype is ctypes.c_int


def test_bytes_per_launch():
    from gradients_taco_compress_amd import abtime
    n, B = 8192 * 2560, 128
    assert abtime.bytes_per_launch("compress", n, B) == 3 * n + 8 * (n // B)
    assert abtime.bytes_per_launch("decompress", n, B) == 3 * n + 8 * (n // B)
    assert abtime.bytes_per_launch("accumulate", n, B) == 9 * n + 8 * (n // B)


@pytest.mark.parametrize("argv", [["x.so", "--ops", "compress,fwht"], ["x.so", "--ops", ","],
                                  ["x.so", "--repeats", "0"], ["x.so", "--workload", "nope"]])
def test_bad_arguments_exit(argv):
    from gradients_taco_compress_amd import abtime
    with pytest.raises(SystemExit) as e:
        abtime.main(argv)
    assert e.value.code == 2
