"""Python binding of libtaco (the TACO FP8 compression operator on MI355X).

The binding only marshals arguments: every step of the operator runs in the
HIP kernels of ``libtaco.so``.  PyTorch provides device memory and the
stream; there is no CPU fallback, and importing this package fails loudly if
the library has not been built (``python -m gradients_taco_compress_amd.build``).

Two layers:

* ``taco_compress``, ``taco_decompress``, ``taco_decompress_accumulate``,
  ``taco_e4m3_encode``, ``taco_e4m3_decode``, ``taco_num_blocks``,
  ``taco_status_string``: the C ABI of ``include/taco.h`` with the same
  names and arguments (device pointers as ints, stream handle as int).
* ``compress``, ``decompress``, ``decompress_accumulate``, ``e4m3_encode``,
  ``e4m3_decode``: the same calls on torch tensors, allocating outputs when
  none are given and launching on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtaco.so")

#: Values fixed by the library (see include/taco.h).
QMAX = 448.0
EPS = 1e-20
BLOCKS = (32, 64, 128, 256, 512)
DEFAULT_TARGET_ENERGY = 1.0

STATUS = {
    0: "TACO_OK", 1: "TACO_ERR_NULL", 2: "TACO_ERR_SHAPE", 3: "TACO_ERR_BLOCK",
    4: "TACO_ERR_PARAM", 5: "TACO_ERR_ALIGN", 6: "TACO_ERR_ALIAS", 7: "TACO_ERR_HIP",
}


class TacoError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({taco_status_string(status)})")


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libtaco.so is not built ({LIB_PATH} missing); run "
        "`python -m gradients_taco_compress_amd.build` (there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)

_P, _I64, _I32, _F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
_lib.taco_num_blocks.argtypes = [_I64, _I64, _I32]
_lib.taco_num_blocks.restype = _I64
_lib.taco_compress.argtypes = [_P, _I64, _I64, _I32, _F32, _P, _P, _P, _P]
_lib.taco_compress.restype = ctypes.c_int
_lib.taco_decompress.argtypes = [_P, _P, _P, _I64, _I64, _I32, _P, _P]
_lib.taco_decompress.restype = ctypes.c_int
_lib.taco_decompress_accumulate.argtypes = [_P, _P, _P, _I64, _I64, _I32, _P, _P]
_lib.taco_decompress_accumulate.restype = ctypes.c_int
_lib.taco_e4m3_encode.argtypes = [_P, _I64, _P, _P]
_lib.taco_e4m3_encode.restype = ctypes.c_int
_lib.taco_e4m3_decode.argtypes = [_P, _I64, _P, _P]
_lib.taco_e4m3_decode.restype = ctypes.c_int
_lib.taco_status_string.argtypes = [ctypes.c_int]
_lib.taco_status_string.restype = ctypes.c_char_p

#: Symbols the library exports (checked against include/taco.h by the tests).
EXPORTS = ("taco_num_blocks", "taco_compress", "taco_decompress",
           "taco_decompress_accumulate", "taco_e4m3_encode", "taco_e4m3_decode",
           "taco_status_string")


# ------------------------------------------------------------- raw C ABI --

def taco_num_blocks(tokens: int, hidden: int, block: int) -> int:
    return _lib.taco_num_blocks(tokens, hidden, block)


def taco_status_string(status: int) -> str:
    return _lib.taco_status_string(status).decode()


def taco_compress(x_bf16: int, tokens: int, hidden: int, block: int, target_energy: float,
                  codes_e4m3: int, alpha: int, scale: int, stream: int) -> int:
    return _lib.taco_compress(x_bf16, tokens, hidden, block, target_energy, codes_e4m3,
                              alpha, scale, stream)


def taco_decompress(codes_e4m3: int, alpha: int, scale: int, tokens: int, hidden: int,
                    block: int, y_bf16: int, stream: int) -> int:
    return _lib.taco_decompress(codes_e4m3, alpha, scale, tokens, hidden, block, y_bf16, stream)


def taco_decompress_accumulate(codes_e4m3: int, alpha: int, scale: int, tokens: int,
                               hidden: int, block: int, acc_f32: int, stream: int) -> int:
    return _lib.taco_decompress_accumulate(codes_e4m3, alpha, scale, tokens, hidden, block,
                                           acc_f32, stream)


def taco_e4m3_encode(x: int, n: int, codes: int, stream: int) -> int:
    return _lib.taco_e4m3_encode(x, n, codes, stream)


def taco_e4m3_decode(codes: int, n: int, out: int, stream: int) -> int:
    return _lib.taco_e4m3_decode(codes, n, out, stream)


# ---------------------------------------------------------- torch layer --

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _shape2(t):
    """(tokens, hidden) of a tensor: the last dim is hidden."""
    if t.dim() == 0:
        raise ValueError("expected a tensor with at least one dimension")
    hidden = t.shape[-1]
    tokens = t.numel() // hidden if hidden else 0
    return tokens, hidden


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(status: int, what: str):
    if status != 0:
        raise TacoError(status, what)


def compress(x, block: int = 256, target_energy: float = DEFAULT_TARGET_ENERGY,
             codes=None, alpha=None, scale=None, stream=None):
    """Compress a bf16 tensor [..., hidden]: returns (codes uint8 same shape,
    alpha float32 [M], scale float32 [M])."""
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    tokens, hidden = _shape2(x)
    m = taco_num_blocks(tokens, hidden, block)
    if m < 0:   # let the library name the validation error
        _check(taco_compress(x.data_ptr(), tokens, hidden, block, float(target_energy),
                             0, 0, 0, _stream(stream)), "taco_compress")
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if alpha is None:
        alpha = torch.empty(m, dtype=torch.float32, device=x.device)
    if scale is None:
        scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(alpha, torch.float32, "alpha")
    _need(scale, torch.float32, "scale")
    if codes.numel() != x.numel() or alpha.numel() < m or scale.numel() < m:
        raise ValueError("output buffers are too small")
    _check(taco_compress(x.data_ptr(), tokens, hidden, block, float(target_energy),
                         codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), _stream(stream)),
           "taco_compress")
    return codes, alpha, scale


def _receiver_args(codes, alpha, scale, block):
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    _need(alpha, torch.float32, "alpha")
    _need(scale, torch.float32, "scale")
    tokens, hidden = _shape2(codes)
    m = taco_num_blocks(tokens, hidden, block)
    if m >= 0 and (alpha.numel() < m or scale.numel() < m):
        raise ValueError("alpha / scale hold fewer than numel / block entries")
    return tokens, hidden


def decompress(codes, alpha, scale, block: int = 256, out=None, stream=None):
    """Reconstruct a bf16 tensor with the shape of ``codes``."""
    torch = _torch()
    tokens, hidden = _receiver_args(codes, alpha, scale, block)
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    _need(out, torch.bfloat16, "out")
    if out.numel() != codes.numel():
        raise ValueError("out must have as many elements as codes")
    _check(taco_decompress(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), tokens, hidden,
                           block, out.data_ptr(), _stream(stream)), "taco_decompress")
    return out


def decompress_accumulate(codes, alpha, scale, acc, block: int = 256, stream=None):
    """acc (float32, same number of elements as codes) += reconstruction."""
    torch = _torch()
    tokens, hidden = _receiver_args(codes, alpha, scale, block)
    _need(acc, torch.float32, "acc")
    if acc.numel() != codes.numel():
        raise ValueError("acc must have as many elements as codes")
    _check(taco_decompress_accumulate(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), tokens,
                                      hidden, block, acc.data_ptr(), _stream(stream)),
           "taco_decompress_accumulate")
    return acc


def e4m3_encode(x, out=None, stream=None):
    """Element-wise E4M3 codes of a float32 tensor (the kernels' conversion)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    _check(taco_e4m3_encode(x.data_ptr(), x.numel(), out.data_ptr(), _stream(stream)),
           "taco_e4m3_encode")
    return out


def e4m3_decode(codes, out=None, stream=None):
    """Element-wise float32 values of E4M3 codes (the kernels' conversion)."""
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _need(out, torch.float32, "out")
    _check(taco_e4m3_decode(codes.data_ptr(), codes.numel(), out.data_ptr(), _stream(stream)),
           "taco_e4m3_decode")
    return out
