"""Binding of libtaco_probe (include/taco_probe.h): an empty kernel and plain
streaming kernels with the byte mixes of libtaco's kernels, used by the
benchmark to measure the launch floor and the streaming ceiling at each
tensor size.  Not part of the operator."""
from __future__ import annotations

import ctypes
import os

from . import _torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtaco_probe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run python gradients_taco_compress_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)
_lib.taco_probe_empty.argtypes = [ctypes.c_int64, ctypes.c_void_p]
_lib.taco_probe_empty.restype = ctypes.c_int
_lib.taco_probe_stream.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_void_p]
_lib.taco_probe_stream.restype = ctypes.c_int

#: Symbols the library exports (checked against include/taco_probe.h).
EXPORTS = ("taco_probe_empty", "taco_probe_stream")
#: (loads, stores) KiB per wavefront of the byte mixes: compress at B = 128,
#: decompress, accumulate, copy.
MIXES = {"compress": (2, 1), "decompress": (1, 2), "accumulate": (5, 4), "copy": (1, 1)}


def taco_probe_empty(groups: int, stream: int) -> int:
    return _lib.taco_probe_empty(groups, stream)


def taco_probe_stream(loads: int, stores: int, valu: int, src: int, dst: int, waves: int,
                      stream: int) -> int:
    return _lib.taco_probe_stream(loads, stores, valu, src, dst, waves, stream)


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def empty(groups: int) -> None:
    """Launch the empty kernel on `groups` work-groups (torch's current stream)."""
    st = taco_probe_empty(groups, _stream())
    if st != 0:
        raise RuntimeError(f"taco_probe_empty failed ({st})")


def stream(mix: str, src, dst, waves: int, valu: int = 0) -> None:
    """One plain stream of a byte mix over `waves` wavefronts (with `valu`
    dependent VALU instructions per wavefront between loads and stores): src
    and dst are device tensors of at least waves * loads and waves * stores
    KiB."""
    ld, sto = MIXES[mix]
    if src.numel() * src.element_size() < waves * ld * 1024 or \
            dst.numel() * dst.element_size() < waves * sto * 1024:
        raise ValueError("buffers too small for the stream")
    st = taco_probe_stream(ld, sto, valu, src.data_ptr(), dst.data_ptr(), waves, _stream())
    if st != 0:
        raise RuntimeError(f"taco_probe_stream failed ({st})")
