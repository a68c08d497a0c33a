"""Python binding of libtaco (the TACO FP8 compression operator on MI355X).

The binding only marshals arguments: every step of the operator runs in the
HIP kernels of ``libtaco.so``.  PyTorch provides device memory and the
stream; there is no CPU fallback, and importing this package fails loudly if
the library has not been built (``python gradients_taco_compress_amd/build.py``).

Two layers:

* ``taco_compress``, ``taco_decompress``, ``taco_decompress_accumulate``,
  ``taco_reduce_compress``, their ``*_packed`` forms, the ``*_fmt`` forms of
  all eight (with a code format), ``taco_packed_bytes``, ``taco_encode``,
  ``taco_decode``, ``taco_e4m3_encode``, ``taco_e4m3_decode``,
  ``taco_roundtrip``, ``taco_roundtrip_noalloc``, ``taco_num_blocks``,
  ``taco_status_string``: the C ABI of
  ``include/taco.h`` with the same names and arguments (device pointers as
  ints, stream handle as int, pointer arrays as sequences of ints, formats
  as the ints of ``FORMATS``).
* ``compress``, ``decompress``, ``decompress_accumulate``, ``reduce_compress``,
  their ``*_packed`` forms on interleaved payloads, ``encode``, ``decode``,
  ``e4m3_encode``, ``e4m3_decode``, ``roundtrip`` (with ``fidelity_metrics``):
  the same calls on torch tensors,
  allocating outputs when none are given and launching on torch's current
  stream.  ``fmt`` names the code format ("e4m3", "e5m2" or "int8"); E4M3
  goes through the entry points without a format.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtaco.so")

#: Values fixed by the library (see include/taco.h).
QMAX = 448.0
#: Code formats (taco_format) and their Q_max.
FORMATS = {"e4m3": 0, "e5m2": 1, "int8": 2}
QMAX_OF = {"e4m3": 448.0, "e5m2": 57344.0, "int8": 127.0}
#: Round-trip variants of the fidelity study (taco_variant).
VARIANTS = {"taco": 0, "direct": 1, "ds": 2, "ash": 3, "hadamard": 4, "tensor": 5}
EPS = 1e-20
BLOCKS = (32, 64, 128, 256, 512)
DEFAULT_TARGET_ENERGY = 1.0

STATUS = {
    0: "TACO_OK", 1: "TACO_ERR_NULL", 2: "TACO_ERR_SHAPE", 3: "TACO_ERR_BLOCK",
    4: "TACO_ERR_PARAM", 5: "TACO_ERR_ALIGN", 6: "TACO_ERR_ALIAS", 7: "TACO_ERR_HIP",
    8: "TACO_ERR_FORMAT",
}


class TacoError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({taco_status_string(status)})")


# libtaco.so names the HIP runtime by its soname (libamdhip64.so.7).  torch
# ships its own copy of that runtime and loads it by another name, so which
# copy the library binds to depends on load order: loading torch first makes
# libtaco use torch's runtime, for which torch's device pointers and stream
# handles are valid.  (Loaded the other way round, the process holds two HIP
# runtimes and every launch on a torch stream fails.)
try:
    import torch as _torch_first  # noqa: F401
except ImportError:  # pragma: no cover - the C ABI itself needs no torch
    pass

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libtaco.so is not built ({LIB_PATH} missing); run "
        "`python gradients_taco_compress_amd/build.py` (there is no CPU fallback)")

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
_lib.taco_reduce_compress.argtypes = [_P, _I32, _P, _P, _P, _I64, _I64, _I32, _F32, _P, _P, _P, _P]
_lib.taco_reduce_compress.restype = ctypes.c_int
_lib.taco_packed_bytes.argtypes = [_I64, _I64, _I32]
_lib.taco_packed_bytes.restype = _I64
_lib.taco_compress_packed.argtypes = [_P, _I64, _I64, _I32, _F32, _P, _P]
_lib.taco_compress_packed.restype = ctypes.c_int
_lib.taco_decompress_packed.argtypes = [_P, _I64, _I64, _I32, _P, _P]
_lib.taco_decompress_packed.restype = ctypes.c_int
_lib.taco_decompress_accumulate_packed.argtypes = [_P, _I64, _I64, _I32, _P, _P]
_lib.taco_decompress_accumulate_packed.restype = ctypes.c_int
_lib.taco_reduce_compress_packed.argtypes = [_P, _I32, _P, _I64, _I64, _I32, _F32, _P, _P]
_lib.taco_reduce_compress_packed.restype = ctypes.c_int
_lib.taco_e4m3_encode.argtypes = [_P, _I64, _P, _P]
_lib.taco_e4m3_encode.restype = ctypes.c_int
_lib.taco_e4m3_decode.argtypes = [_P, _I64, _P, _P]
_lib.taco_e4m3_decode.restype = ctypes.c_int
_lib.taco_compress_fmt.argtypes = [_P, _I64, _I64, _I32, _F32, _I32, _P, _P, _P, _P]
_lib.taco_decompress_fmt.argtypes = [_P, _P, _P, _I64, _I64, _I32, _I32, _P, _P]
_lib.taco_decompress_accumulate_fmt.argtypes = [_P, _P, _P, _I64, _I64, _I32, _I32, _P, _P]
_lib.taco_reduce_compress_fmt.argtypes = [_P, _I32, _P, _P, _P, _I64, _I64, _I32, _F32, _I32,
                                          _P, _P, _P, _P]
_lib.taco_compress_packed_fmt.argtypes = [_P, _I64, _I64, _I32, _F32, _I32, _P, _P]
_lib.taco_decompress_packed_fmt.argtypes = [_P, _I64, _I64, _I32, _I32, _P, _P]
_lib.taco_decompress_accumulate_packed_fmt.argtypes = [_P, _I64, _I64, _I32, _I32, _P, _P]
_lib.taco_reduce_compress_packed_fmt.argtypes = [_P, _I32, _P, _I64, _I64, _I32, _F32, _I32,
                                                 _P, _P]
_lib.taco_decompress_accumulate_n.argtypes = [_I32, _P, _P, _P, _I64, _I64, _I32, _P, _P]
_lib.taco_decompress_accumulate_n_fmt.argtypes = [_I32, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P]
_lib.taco_decompress_accumulate_n_packed.argtypes = [_I32, _P, _I64, _I64, _I32, _P, _P]
_lib.taco_decompress_accumulate_n_packed_fmt.argtypes = [_I32, _P, _I64, _I64, _I32, _I32, _P, _P]
for _name in ("decompress_accumulate_n", "decompress_accumulate_n_fmt",
              "decompress_accumulate_n_packed", "decompress_accumulate_n_packed_fmt"):
    getattr(_lib, "taco_" + _name).restype = ctypes.c_int
_lib.taco_roundtrip.argtypes = [_P, _I64, _I64, _I32, _F32, _I32, _I32, _P, _P, _P]
_lib.taco_roundtrip.restype = ctypes.c_int
_lib.taco_roundtrip_noalloc.argtypes = [_P, _I64, _I64, _I32, _F32, _I32, _I32, _P, _P, _P]
_lib.taco_roundtrip_noalloc.restype = ctypes.c_int
_lib.taco_encode.argtypes = [_I32, _P, _I64, _P, _P]
_lib.taco_decode.argtypes = [_I32, _P, _I64, _P, _P]
for _name in ("compress_fmt", "decompress_fmt", "decompress_accumulate_fmt",
              "reduce_compress_fmt", "compress_packed_fmt", "decompress_packed_fmt",
              "decompress_accumulate_packed_fmt", "reduce_compress_packed_fmt", "encode",
              "decode"):
    getattr(_lib, "taco_" + _name).restype = ctypes.c_int
_lib.taco_status_string.argtypes = [ctypes.c_int]
_lib.taco_status_string.restype = ctypes.c_char_p

#: Symbols the library exports (checked against include/taco.h by the tests).
EXPORTS = ("taco_num_blocks", "taco_compress", "taco_decompress",
           "taco_decompress_accumulate", "taco_reduce_compress", "taco_packed_bytes",
           "taco_compress_packed", "taco_decompress_packed", "taco_decompress_accumulate_packed",
           "taco_reduce_compress_packed", "taco_e4m3_encode", "taco_e4m3_decode",
           "taco_status_string", "taco_compress_fmt", "taco_decompress_fmt",
           "taco_decompress_accumulate_fmt", "taco_reduce_compress_fmt",
           "taco_compress_packed_fmt", "taco_decompress_packed_fmt",
           "taco_decompress_accumulate_packed_fmt", "taco_reduce_compress_packed_fmt",
           "taco_encode", "taco_decode", "taco_roundtrip", "taco_decompress_accumulate_n",
           "taco_decompress_accumulate_n_fmt", "taco_decompress_accumulate_n_packed",
           "taco_decompress_accumulate_n_packed_fmt", "taco_roundtrip_noalloc")

#: Most payloads one taco_reduce_compress or taco_decompress_accumulate_n
#: call sums.
MAX_PAYLOADS = 8


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


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*[int(p) for p in ptrs])
    return arr


def taco_reduce_compress(own_bf16: int, npayloads: int, codes_e4m3, alpha, scale, tokens: int,
                         hidden: int, block: int, target_energy: float, out_codes: int,
                         out_alpha: int, out_scale: int, stream: int) -> int:
    """codes_e4m3 / alpha / scale: sequences of npayloads device pointers
    (passed to the library as host arrays), or None when npayloads is 0."""
    arrs = [None if a is None else _ptr_array(a) for a in (codes_e4m3, alpha, scale)]
    args = [None if a is None else ctypes.cast(a, ctypes.c_void_p) for a in arrs]
    return _lib.taco_reduce_compress(own_bf16, npayloads, args[0], args[1], args[2], tokens,
                                     hidden, block, target_energy, out_codes, out_alpha,
                                     out_scale, stream)


def taco_packed_bytes(tokens: int, hidden: int, block: int) -> int:
    return _lib.taco_packed_bytes(tokens, hidden, block)


def taco_compress_packed(x_bf16: int, tokens: int, hidden: int, block: int, target_energy: float,
                         payload: int, stream: int) -> int:
    return _lib.taco_compress_packed(x_bf16, tokens, hidden, block, target_energy, payload, stream)


def taco_decompress_packed(payload: int, tokens: int, hidden: int, block: int, y_bf16: int,
                           stream: int) -> int:
    return _lib.taco_decompress_packed(payload, tokens, hidden, block, y_bf16, stream)


def taco_decompress_accumulate_packed(payload: int, tokens: int, hidden: int, block: int,
                                      acc_f32: int, stream: int) -> int:
    return _lib.taco_decompress_accumulate_packed(payload, tokens, hidden, block, acc_f32, stream)


def taco_reduce_compress_packed(own_bf16: int, npayloads: int, payloads, tokens: int, hidden: int,
                                block: int, target_energy: float, out_payload: int,
                                stream: int) -> int:
    """payloads: sequence of npayloads device pointers (a host array), or None."""
    arr = None if payloads is None else ctypes.cast(_ptr_array(payloads), ctypes.c_void_p)
    return _lib.taco_reduce_compress_packed(own_bf16, npayloads, arr, tokens, hidden, block,
                                            target_energy, out_payload, stream)


def taco_compress_fmt(x_bf16: int, tokens: int, hidden: int, block: int, target_energy: float,
                      format: int, codes: int, alpha: int, scale: int, stream: int) -> int:
    return _lib.taco_compress_fmt(x_bf16, tokens, hidden, block, target_energy, format, codes,
                                  alpha, scale, stream)


def taco_decompress_fmt(codes: int, alpha: int, scale: int, tokens: int, hidden: int, block: int,
                        format: int, y_bf16: int, stream: int) -> int:
    return _lib.taco_decompress_fmt(codes, alpha, scale, tokens, hidden, block, format, y_bf16,
                                    stream)


def taco_decompress_accumulate_fmt(codes: int, alpha: int, scale: int, tokens: int, hidden: int,
                                   block: int, format: int, acc_f32: int, stream: int) -> int:
    return _lib.taco_decompress_accumulate_fmt(codes, alpha, scale, tokens, hidden, block, format,
                                               acc_f32, stream)


def taco_reduce_compress_fmt(own_bf16: int, npayloads: int, codes, alpha, scale, tokens: int,
                             hidden: int, block: int, target_energy: float, format: int,
                             out_codes: int, out_alpha: int, out_scale: int, stream: int) -> int:
    arrs = [None if a is None else _ptr_array(a) for a in (codes, alpha, scale)]
    args = [None if a is None else ctypes.cast(a, ctypes.c_void_p) for a in arrs]
    return _lib.taco_reduce_compress_fmt(own_bf16, npayloads, args[0], args[1], args[2], tokens,
                                         hidden, block, target_energy, format, out_codes,
                                         out_alpha, out_scale, stream)


def taco_compress_packed_fmt(x_bf16: int, tokens: int, hidden: int, block: int,
                             target_energy: float, format: int, payload: int,
                             stream: int) -> int:
    return _lib.taco_compress_packed_fmt(x_bf16, tokens, hidden, block, target_energy, format,
                                         payload, stream)


def taco_decompress_packed_fmt(payload: int, tokens: int, hidden: int, block: int, format: int,
                               y_bf16: int, stream: int) -> int:
    return _lib.taco_decompress_packed_fmt(payload, tokens, hidden, block, format, y_bf16, stream)


def taco_decompress_accumulate_packed_fmt(payload: int, tokens: int, hidden: int, block: int,
                                          format: int, acc_f32: int, stream: int) -> int:
    return _lib.taco_decompress_accumulate_packed_fmt(payload, tokens, hidden, block, format,
                                                      acc_f32, stream)


def taco_reduce_compress_packed_fmt(own_bf16: int, npayloads: int, payloads, tokens: int,
                                    hidden: int, block: int, target_energy: float, format: int,
                                    out_payload: int, stream: int) -> int:
    arr = None if payloads is None else ctypes.cast(_ptr_array(payloads), ctypes.c_void_p)
    return _lib.taco_reduce_compress_packed_fmt(own_bf16, npayloads, arr, tokens, hidden, block,
                                                target_energy, format, out_payload, stream)


def taco_encode(format: int, x: int, n: int, codes: int, stream: int) -> int:
    return _lib.taco_encode(format, x, n, codes, stream)


def taco_decode(format: int, codes: int, n: int, out: int, stream: int) -> int:
    return _lib.taco_decode(format, codes, n, out, stream)


def _arr(ptrs):
    return None if ptrs is None else ctypes.cast(_ptr_array(ptrs), ctypes.c_void_p)


def taco_decompress_accumulate_n(npayloads: int, codes_e4m3, alpha, scale, tokens: int,
                                 hidden: int, block: int, acc_f32: int, stream: int) -> int:
    return _lib.taco_decompress_accumulate_n(npayloads, _arr(codes_e4m3), _arr(alpha),
                                             _arr(scale), tokens, hidden, block, acc_f32, stream)


def taco_decompress_accumulate_n_fmt(npayloads: int, codes, alpha, scale, tokens: int,
                                     hidden: int, block: int, format: int, acc_f32: int,
                                     stream: int) -> int:
    return _lib.taco_decompress_accumulate_n_fmt(npayloads, _arr(codes), _arr(alpha), _arr(scale),
                                                 tokens, hidden, block, format, acc_f32, stream)


def taco_decompress_accumulate_n_packed(npayloads: int, payloads, tokens: int, hidden: int,
                                        block: int, acc_f32: int, stream: int) -> int:
    return _lib.taco_decompress_accumulate_n_packed(npayloads, _arr(payloads), tokens, hidden,
                                                    block, acc_f32, stream)


def taco_decompress_accumulate_n_packed_fmt(npayloads: int, payloads, tokens: int, hidden: int,
                                            block: int, format: int, acc_f32: int,
                                            stream: int) -> int:
    return _lib.taco_decompress_accumulate_n_packed_fmt(npayloads, _arr(payloads), tokens, hidden,
                                                        block, format, acc_f32, stream)


def taco_roundtrip(x_bf16: int, tokens: int, hidden: int, block: int, target_energy: float,
                   format: int, variant: int, y_bf16: int, sums: int, stream: int) -> int:
    return _lib.taco_roundtrip(x_bf16, tokens, hidden, block, target_energy, format, variant,
                               y_bf16, sums, stream)


def taco_roundtrip_noalloc(x_bf16: int, tokens: int, hidden: int, block: int,
                           target_energy: float, format: int, variant: int, y_bf16: int,
                           totals: int, stream: int) -> int:
    return _lib.taco_roundtrip_noalloc(x_bf16, tokens, hidden, block, target_energy, format,
                                       variant, y_bf16, totals, stream)


def taco_e4m3_encode(x: int, n: int, codes: int, stream: int) -> int:
    return _lib.taco_e4m3_encode(x, n, codes, stream)


def taco_e4m3_decode(codes: int, n: int, out: int, stream: int) -> int:
    return _lib.taco_e4m3_decode(codes, n, out, stream)


# ---------------------------------------------------------- torch layer --

def _torch():
    import torch
    return torch


def _stream(stream, *tensors):
    """Handle of the stream to launch on: ``stream``, else torch's current
    stream of the device the tensors live on.  Every tensor (None entries and
    nested lists allowed) must be on that one device."""
    torch = _torch()
    devs = set()
    todo = list(tensors)
    while todo:
        t = todo.pop()
        if t is None:
            continue
        if isinstance(t, (list, tuple)):
            todo.extend(t)
            continue
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(str(d) for d in devs)}")
    dev = next(iter(devs)) if devs else None
    s = torch.cuda.current_stream(dev) if stream is None else stream
    if dev is not None and s.device != dev:
        raise ValueError(f"stream is on {s.device}, tensors on {dev}")
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


def _format(fmt: str) -> int:
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown code format {fmt!r} (one of {sorted(FORMATS)})") from None


def _compress_call(fmt, x, tokens, hidden, block, tau, codes, alpha, scale, stream):
    if fmt == "e4m3":
        return taco_compress(x, tokens, hidden, block, tau, codes, alpha, scale, stream)
    return taco_compress_fmt(x, tokens, hidden, block, tau, _format(fmt), codes, alpha, scale,
                             stream)


def compress(x, block: int = 256, target_energy: float = DEFAULT_TARGET_ENERGY,
             codes=None, alpha=None, scale=None, stream=None, fmt: str = "e4m3"):
    """Compress a bf16 tensor [..., hidden]: returns (codes uint8 same shape,
    alpha float32 [M], scale float32 [M])."""
    torch = _torch()
    _format(fmt)
    _need(x, torch.bfloat16, "x")
    tokens, hidden = _shape2(x)
    m = taco_num_blocks(tokens, hidden, block)
    if m < 0:   # let the library name the validation error
        _check(_compress_call(fmt, x.data_ptr(), tokens, hidden, block, float(target_energy),
                              0, 0, 0, _stream(stream, x)), "taco_compress")
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
    _check(_compress_call(fmt, x.data_ptr(), tokens, hidden, block, float(target_energy),
                          codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), _stream(stream, x, codes, alpha, scale)),
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


def decompress(codes, alpha, scale, block: int = 256, out=None, stream=None, fmt: str = "e4m3"):
    """Reconstruct a bf16 tensor with the shape of ``codes``."""
    torch = _torch()
    f = _format(fmt)
    tokens, hidden = _receiver_args(codes, alpha, scale, block)
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    _need(out, torch.bfloat16, "out")
    if out.numel() != codes.numel():
        raise ValueError("out must have as many elements as codes")
    if fmt == "e4m3":
        st = taco_decompress(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), tokens, hidden,
                             block, out.data_ptr(), _stream(stream, codes, alpha, scale, out))
    else:
        st = taco_decompress_fmt(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), tokens,
                                 hidden, block, f, out.data_ptr(), _stream(stream, codes, alpha, scale, out))
    _check(st, "taco_decompress")
    return out


def decompress_accumulate(codes, alpha, scale, acc, block: int = 256, stream=None,
                          fmt: str = "e4m3"):
    """acc (float32, same number of elements as codes) += reconstruction."""
    torch = _torch()
    f = _format(fmt)
    tokens, hidden = _receiver_args(codes, alpha, scale, block)
    _need(acc, torch.float32, "acc")
    if acc.numel() != codes.numel():
        raise ValueError("acc must have as many elements as codes")
    if fmt == "e4m3":
        st = taco_decompress_accumulate(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(),
                                        tokens, hidden, block, acc.data_ptr(), _stream(stream, codes, alpha, scale, acc))
    else:
        st = taco_decompress_accumulate_fmt(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(),
                                            tokens, hidden, block, f, acc.data_ptr(),
                                            _stream(stream, codes, alpha, scale, acc))
    _check(st, "taco_decompress_accumulate")
    return acc


def reduce_compress(own, payloads, block: int = 256, target_energy: float = DEFAULT_TARGET_ENERGY,
                    codes=None, alpha=None, scale=None, stream=None, fmt: str = "e4m3"):
    """Owner step: compress own + the sum of the payloads' reconstructions.
    own: bf16 tensor or None; payloads: list of (codes, alpha, scale) as
    returned by compress() with the same format.  Returns (codes, alpha,
    scale)."""
    torch = _torch()
    f = _format(fmt)
    ref = own if own is not None else (payloads[0][0] if payloads else None)
    if ref is None:
        raise ValueError("need own or at least one payload")
    if own is not None:
        _need(own, torch.bfloat16, "own")
    tokens, hidden = _shape2(ref)
    for c, a, s in payloads:
        _need(c, torch.uint8, "payload codes")
        _need(a, torch.float32, "payload alpha")
        _need(s, torch.float32, "payload scale")
        if c.numel() != ref.numel():
            raise ValueError("every payload must have as many codes as own has elements")
    m = taco_num_blocks(tokens, hidden, block)
    if m < 0:
        m = 0
    if codes is None:
        codes = torch.empty(ref.shape, dtype=torch.uint8, device=ref.device)
    if alpha is None:
        alpha = torch.empty(m, dtype=torch.float32, device=ref.device)
    if scale is None:
        scale = torch.empty(m, dtype=torch.float32, device=ref.device)
    _need(codes, torch.uint8, "codes")
    _need(alpha, torch.float32, "alpha")
    _need(scale, torch.float32, "scale")
    for _, a, s in payloads:
        if a.numel() < m or s.numel() < m:
            raise ValueError("payload alpha / scale hold fewer than numel / block entries")
    if codes.numel() != ref.numel() or alpha.numel() < m or scale.numel() < m:
        raise ValueError("output buffers are too small")
    n = len(payloads)
    args = (0 if own is None else own.data_ptr(), n,
            [c.data_ptr() for c, _, _ in payloads] if n else None,
            [a.data_ptr() for _, a, _ in payloads] if n else None,
            [s.data_ptr() for _, _, s in payloads] if n else None,
            tokens, hidden, block, float(target_energy))
    outs = (codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), _stream(stream, own, codes, alpha, scale, payloads))
    if fmt == "e4m3":
        st = taco_reduce_compress(*args, *outs)
    else:
        st = taco_reduce_compress_fmt(*args, f, *outs)
    _check(st, "taco_reduce_compress")
    return codes, alpha, scale


def _packed_len(tokens, hidden, block):
    nb = taco_packed_bytes(tokens, hidden, block)
    if nb < 0:
        raise TacoError(2 if block in BLOCKS else 3, "taco_packed_bytes")
    return nb


def compress_packed(x, block: int = 256, target_energy: float = DEFAULT_TARGET_ENERGY,
                    payload=None, stream=None, fmt: str = "e4m3"):
    """Compress a bf16 tensor into one interleaved payload (uint8, 1-D)."""
    torch = _torch()
    f = _format(fmt)
    _need(x, torch.bfloat16, "x")
    tokens, hidden = _shape2(x)
    nb = _packed_len(tokens, hidden, block)
    if payload is None:
        payload = torch.empty(nb, dtype=torch.uint8, device=x.device)
    _need(payload, torch.uint8, "payload")
    if payload.numel() < nb:
        raise ValueError("payload buffer is too small")
    if fmt == "e4m3":
        st = taco_compress_packed(x.data_ptr(), tokens, hidden, block, float(target_energy),
                                  payload.data_ptr(), _stream(stream, x, payload))
    else:
        st = taco_compress_packed_fmt(x.data_ptr(), tokens, hidden, block, float(target_energy),
                                      f, payload.data_ptr(), _stream(stream, x, payload))
    _check(st, "taco_compress_packed")
    return payload


def decompress_packed(payload, shape, block: int = 256, out=None, stream=None,
                      fmt: str = "e4m3"):
    """Reconstruct a bf16 tensor of the given shape from an interleaved payload."""
    torch = _torch()
    f = _format(fmt)
    _need(payload, torch.uint8, "payload")
    hidden = shape[-1]
    tokens = 1
    for d in shape[:-1]:
        tokens *= d
    if payload.numel() < _packed_len(tokens, hidden, block):
        raise ValueError("payload is too small for this shape")
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=payload.device)
    _need(out, torch.bfloat16, "out")
    if out.numel() != tokens * hidden:
        raise ValueError("out must have as many elements as the shape")
    if fmt == "e4m3":
        st = taco_decompress_packed(payload.data_ptr(), tokens, hidden, block, out.data_ptr(),
                                    _stream(stream, payload, out))
    else:
        st = taco_decompress_packed_fmt(payload.data_ptr(), tokens, hidden, block, f,
                                        out.data_ptr(), _stream(stream, payload, out))
    _check(st, "taco_decompress_packed")
    return out


def decompress_accumulate_packed(payload, acc, block: int = 256, stream=None, fmt: str = "e4m3"):
    """acc (float32) += reconstruction of an interleaved payload."""
    torch = _torch()
    f = _format(fmt)
    _need(payload, torch.uint8, "payload")
    _need(acc, torch.float32, "acc")
    tokens, hidden = _shape2(acc)
    if payload.numel() < _packed_len(tokens, hidden, block):
        raise ValueError("payload is too small for acc's shape")
    if fmt == "e4m3":
        st = taco_decompress_accumulate_packed(payload.data_ptr(), tokens, hidden, block,
                                               acc.data_ptr(), _stream(stream, payload, acc))
    else:
        st = taco_decompress_accumulate_packed_fmt(payload.data_ptr(), tokens, hidden, block, f,
                                                   acc.data_ptr(), _stream(stream, payload, acc))
    _check(st, "taco_decompress_accumulate_packed")
    return acc


def reduce_compress_packed(own, payloads, shape=None, block: int = 256,
                           target_energy: float = DEFAULT_TARGET_ENERGY, out=None, stream=None,
                           fmt: str = "e4m3"):
    """Owner step on interleaved payloads: returns one interleaved payload."""
    torch = _torch()
    f = _format(fmt)
    if own is not None:
        _need(own, torch.bfloat16, "own")
        shape = own.shape
    if shape is None:
        raise ValueError("shape is required without own")
    hidden = shape[-1]
    tokens = 1
    for d in shape[:-1]:
        tokens *= d
    nb = _packed_len(tokens, hidden, block)
    for p in payloads:
        _need(p, torch.uint8, "payload")
        if p.numel() < nb:
            raise ValueError("payload is too small for this shape")
    dev = own.device if own is not None else payloads[0].device
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=dev)
    _need(out, torch.uint8, "out")
    if out.numel() < nb:
        raise ValueError("out is too small for this shape's payload")
    n = len(payloads)
    args = (0 if own is None else own.data_ptr(), n,
            [p.data_ptr() for p in payloads] if n else None, tokens, hidden, block,
            float(target_energy))
    if fmt == "e4m3":
        st = taco_reduce_compress_packed(*args, out.data_ptr(), _stream(stream, own, out, payloads))
    else:
        st = taco_reduce_compress_packed_fmt(*args, f, out.data_ptr(), _stream(stream, own, out, payloads))
    _check(st, "taco_reduce_compress_packed")
    return out


def e4m3_encode(x, out=None, stream=None):
    """Element-wise E4M3 codes of a float32 tensor (the kernels' conversion)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    _check(taco_e4m3_encode(x.data_ptr(), x.numel(), out.data_ptr(), _stream(stream, x, out)),
           "taco_e4m3_encode")
    return out


def e4m3_decode(codes, out=None, stream=None):
    """Element-wise float32 values of E4M3 codes (the kernels' conversion)."""
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _need(out, torch.float32, "out")
    if out.numel() != codes.numel():
        raise ValueError("out must have as many elements as codes")
    _check(taco_e4m3_decode(codes.data_ptr(), codes.numel(), out.data_ptr(), _stream(stream, codes, out)),
           "taco_e4m3_decode")
    return out


def encode(x, fmt: str = "e4m3", out=None, stream=None):
    """Element-wise codes of a float32 tensor in a format (the kernels' conversion)."""
    torch = _torch()
    f = _format(fmt)
    _need(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    _check(taco_encode(f, x.data_ptr(), x.numel(), out.data_ptr(), _stream(stream, x, out)), "taco_encode")
    return out


def decode(codes, fmt: str = "e4m3", out=None, stream=None):
    """Element-wise float32 values of codes in a format (the kernels' conversion)."""
    torch = _torch()
    f = _format(fmt)
    _need(codes, torch.uint8, "codes")
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _need(out, torch.float32, "out")
    if out.numel() != codes.numel():
        raise ValueError("out must have as many elements as codes")
    _check(taco_decode(f, codes.data_ptr(), codes.numel(), out.data_ptr(), _stream(stream, codes, out)),
           "taco_decode")
    return out


#: Bytes of taco_fidelity_sums: the totals (four doubles, two floats) and
#: the library's 64 slots of partial sums.
FIDELITY_SUMS_BYTES = 40 + 4 * 64 * 8 + 2 * 64 * 4
#: Bytes of taco_fidelity_totals (the totals alone, laid out as the front of
#: taco_fidelity_sums).
FIDELITY_TOTALS_BYTES = 40


def roundtrip(x, block: int = 256, variant: str = "taco", fmt: str = "e4m3",
              target_energy: float = DEFAULT_TARGET_ENERGY, want_output: bool = False,
              sums=None, out=None, stream=None):
    """One round trip of a fidelity-study variant over a bf16 tensor.
    Returns (y or None, sums): y is the bf16 reconstruction (when wanted or
    ``out`` is given), sums a uint8 device tensor holding taco_fidelity_sums
    (read it with fidelity_metrics)."""
    torch = _torch()
    f = _format(fmt)
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r} (one of {sorted(VARIANTS)})")
    _need(x, torch.bfloat16, "x")
    tokens, hidden = _shape2(x)
    if sums is None:
        sums = torch.empty(FIDELITY_SUMS_BYTES, dtype=torch.uint8, device=x.device)
    _need(sums, torch.uint8, "sums")
    if sums.numel() < FIDELITY_SUMS_BYTES:
        raise ValueError(f"sums must hold {FIDELITY_SUMS_BYTES} bytes")
    if out is None and want_output:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    if out is not None:
        _need(out, torch.bfloat16, "out")
        if out.numel() != x.numel():
            raise ValueError("out must have as many elements as x")
    _check(taco_roundtrip(x.data_ptr(), tokens, hidden, block, float(target_energy), f,
                          VARIANTS[variant], 0 if out is None else out.data_ptr(),
                          sums.data_ptr(), _stream(stream, x, out, sums)), "taco_roundtrip")
    return out, sums


def fidelity_metrics(sums, n: int) -> dict:
    """RelL2, Cos, MaxErr and MSE (GIFT page, Eq. 21) of a round trip over n
    elements, from its sums (synchronises with the device)."""
    import struct
    raw = bytes(sums[:40].cpu().numpy().tobytes())
    se, sr, so, sd, me, tm = struct.unpack("<4d2f", raw)
    return {"rel_l2": (se / sr) ** 0.5 if sr > 0 else se ** 0.5,
            "cos": sd / (sr * so) ** 0.5 if sr > 0 and so > 0 else 0.0,
            "max_err": me, "mse": se / n if n else 0.0,
            "sum_sq_err": se, "sum_sq_ref": sr, "sum_sq_out": so, "sum_dot": sd,
            "tensor_absmax": tm}


def decompress_accumulate_n(payloads, acc, block: int = 256, stream=None, fmt: str = "e4m3"):
    """acc (float32) += the sum of the payloads' reconstructions, in one pass.
    payloads: list of (codes, alpha, scale) as returned by compress()."""
    torch = _torch()
    f = _format(fmt)
    _need(acc, torch.float32, "acc")
    tokens, hidden = _shape2(acc)
    m = taco_num_blocks(tokens, hidden, block)
    for c, a, s in payloads:
        _need(c, torch.uint8, "payload codes")
        _need(a, torch.float32, "payload alpha")
        _need(s, torch.float32, "payload scale")
        if c.numel() != acc.numel() or (m >= 0 and (a.numel() < m or s.numel() < m)):
            raise ValueError("every payload must match acc's shape")
    n = len(payloads)
    args = (n, [c.data_ptr() for c, _, _ in payloads] if n else None,
            [a.data_ptr() for _, a, _ in payloads] if n else None,
            [s.data_ptr() for _, _, s in payloads] if n else None, tokens, hidden, block)
    if fmt == "e4m3":
        st = taco_decompress_accumulate_n(*args, acc.data_ptr(), _stream(stream, acc, payloads))
    else:
        st = taco_decompress_accumulate_n_fmt(*args, f, acc.data_ptr(), _stream(stream, acc, payloads))
    _check(st, "taco_decompress_accumulate_n")
    return acc


def decompress_accumulate_n_packed(payloads, acc, block: int = 256, stream=None,
                                   fmt: str = "e4m3"):
    """acc (float32) += the sum of interleaved payloads' reconstructions."""
    torch = _torch()
    f = _format(fmt)
    _need(acc, torch.float32, "acc")
    tokens, hidden = _shape2(acc)
    nb = _packed_len(tokens, hidden, block)
    for p in payloads:
        _need(p, torch.uint8, "payload")
        if p.numel() < nb:
            raise ValueError("payload is too small for acc's shape")
    n = len(payloads)
    ptrs = [p.data_ptr() for p in payloads] if n else None
    if fmt == "e4m3":
        st = taco_decompress_accumulate_n_packed(n, ptrs, tokens, hidden, block, acc.data_ptr(),
                                                 _stream(stream, acc, payloads))
    else:
        st = taco_decompress_accumulate_n_packed_fmt(n, ptrs, tokens, hidden, block, f,
                                                     acc.data_ptr(), _stream(stream, acc, payloads))
    _check(st, "taco_decompress_accumulate_n_packed")
    return acc
