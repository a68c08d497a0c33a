"""TACO CPU oracle -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``taco_oracle.c`` (plain C, double precision, one
thread).  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package; the GPU library and its Python binding
never do.  What each function computes, and the readings of points the TACO
paper leaves open, are documented in ``taco_oracle.c``.

Arrays are numpy arrays: bf16 tensors travel as ``uint16`` bit patterns,
codes as ``uint8``, alpha / s as ``float32``.

``TACO_ORACLE_MUTANT``, when set, names a build of a deliberately broken
copy of ``taco_oracle.c`` to load instead: ``tests/test_oracle_mutants.py``
uses it to show that the pins catch each planted mistake.  Nothing else sets
it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "taco_oracle.c")
_LIB = os.path.join(_HERE, "libtaco_oracle.so")

#: epsilon of Eq. 6 that the GPU library documents; the oracle takes it as a
#: parameter so tests can vary it.
EPS = 1e-20

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(os.environ.get("TACO_ORACLE_MUTANT") or build())
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.taco_oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.taco_oracle_e4m3_decode.restype = f64
        lib.taco_oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.taco_oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.taco_oracle_double_to_bf16.argtypes = [f64]
        lib.taco_oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.taco_oracle_e4m3_encode_array.argtypes = [P, i64, P]
        lib.taco_oracle_e4m3_encode_array.restype = None
        lib.taco_oracle_e4m3_decode_array.argtypes = [P, i64, P]
        lib.taco_oracle_e4m3_decode_array.restype = None
        lib.taco_oracle_double_to_bf16_array.argtypes = [P, i64, P]
        lib.taco_oracle_double_to_bf16_array.restype = None
        lib.taco_oracle_fwht.argtypes = [P, i32]
        lib.taco_oracle_fwht.restype = None
        lib.taco_oracle_ash_block.argtypes = [P, i32, f64, f64, P, P, P]
        lib.taco_oracle_compress.argtypes = [P, i64, i32, f64, f64, P, P, P]
        lib.taco_oracle_compress_fmt.argtypes = [P, i64, i32, f64, f64, i32, P, P, P]
        lib.taco_oracle_reconstruct_f64.argtypes = [P, P, P, i64, i32, i32, P]
        lib.taco_oracle_decompress.argtypes = [P, P, P, i64, i32, i32, P]
        lib.taco_oracle_decompress_accumulate.argtypes = [P, P, P, i64, i32, i32, P]
        lib.taco_oracle_roundtrip_noquant.argtypes = [P, i32, f64, f64, P]
        lib.taco_oracle_compress_f64.argtypes = [P, i64, i32, f64, f64, i32, P, P, P]
        lib.taco_oracle_reduce_compress.argtypes = [P, i32, P, P, P, i64, i32, f64, f64, i32,
                                                    P, P, P]
        lib.taco_oracle_roundtrip_variant.argtypes = [P, i64, i32, i32, i32, f64, f64, P]
        lib.taco_oracle_fidelity.argtypes = [P, P, i64, P]
        lib.taco_oracle_decompress_accumulate_n.argtypes = [i32, P, P, P, i64, i32, i32, P]
        lib.taco_oracle_qmax.argtypes = [i32]
        lib.taco_oracle_qmax.restype = f64
        lib.taco_oracle_encode_array.argtypes = [i32, P, i64, P]
        lib.taco_oracle_encode_array.restype = None
        lib.taco_oracle_decode_array.argtypes = [i32, P, i64, P]
        lib.taco_oracle_decode_array.restype = None
        for name, arg, res in (("e5m2_decode", ctypes.c_uint8, f64),
                               ("e5m2_encode", ctypes.c_float, ctypes.c_uint8),
                               ("int8_decode", ctypes.c_uint8, f64),
                               ("int8_encode", ctypes.c_float, ctypes.c_uint8)):
            fn = getattr(lib, "taco_oracle_" + name)
            fn.argtypes = [arg]
            fn.restype = res
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise ValueError("oracle rejected the arguments (block must be a power of two "
                         "in [2, 4096] dividing the element count)")


# ---------------------------------------------------------------- codecs ----

#: Code formats: E4M3 (the operator's), E5M2 (section 5.3.2 format ablation)
#: and INT8 (section 6 fallback; section 2.3 / Eq. 1 quantiser).
FORMATS = {"e4m3": 0, "e5m2": 1, "int8": 2}


def _fmt(fmt: str) -> int:
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown code format {fmt!r} (one of {sorted(FORMATS)})") from None


def qmax(fmt: str = "e4m3") -> float:
    """Q_max of Eq. 9 for a code format."""
    return float(_load().taco_oracle_qmax(_fmt(fmt)))


def decode(codes, fmt: str = "e4m3") -> np.ndarray:
    """Values (float64) of codes of a format."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib.taco_oracle_decode_array(_fmt(fmt), _ptr(c), c.size, _ptr(out))
    return out


def encode(values, fmt: str = "e4m3") -> np.ndarray:
    """Nearest-even, saturating codes of float32 values in a format."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib.taco_oracle_encode_array(_fmt(fmt), _ptr(v), v.size, _ptr(out))
    return out


def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib.taco_oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(values) -> np.ndarray:
    """Nearest-even, saturating E4M3 codes of float32 values."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib.taco_oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def double_to_bf16(values) -> np.ndarray:
    """bf16 bit patterns (uint16) of float64 values, nearest-even."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib.taco_oracle_double_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def encode_function_address(fmt: str = "e4m3") -> int:
    """Address of a scalar C encoder (for the exhaustive test helper)."""
    _fmt(fmt)
    return ctypes.cast(getattr(_load(), f"taco_oracle_{fmt}_encode"), ctypes.c_void_p).value


def decode_function_address(fmt: str = "e4m3") -> int:
    """Address of a scalar C decoder (for the exhaustive test helper)."""
    _fmt(fmt)
    return ctypes.cast(getattr(_load(), f"taco_oracle_{fmt}_decode"), ctypes.c_void_p).value


def fwht(v) -> np.ndarray:
    """Unnormalised Sylvester-order FWHT of the last axis (float64 copy)."""
    lib = _load()
    a = np.array(v, dtype=np.float64, copy=True)
    n = a.shape[-1]
    flat = a.reshape(-1, n)
    for row in flat:
        lib.taco_oracle_fwht(_ptr(row), n)
    return flat.reshape(a.shape)


# ------------------------------------------------------------ operator ----

def ash_block(x_bits, block: int, tau: float = 1.0, eps: float = EPS):
    """(alpha, Gt, Z) in float64 for one block of bf16 bit patterns."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    assert x.size == block
    alpha = np.zeros(1, np.float64)
    gt = np.zeros(block, np.float64)
    z = np.zeros(block, np.float64)
    _check(lib.taco_oracle_ash_block(_ptr(x), block, tau, eps, _ptr(alpha), _ptr(gt), _ptr(z)))
    return float(alpha[0]), gt, z


def compress(x_bits, block: int, tau: float = 1.0, eps: float = EPS, fmt: str = "e4m3"):
    """Codes (uint8, same shape as x), alpha and s (float32, one per block)."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    n = x.size
    if block <= 0 or n % block:
        raise ValueError("element count must be a multiple of the block size")
    codes = np.empty(x.shape, np.uint8)
    alpha = np.empty(n // block, np.float32)
    scale = np.empty(n // block, np.float32)
    _check(lib.taco_oracle_compress_fmt(_ptr(x), n, block, tau, eps, _fmt(fmt), _ptr(codes),
                                        _ptr(alpha), _ptr(scale)))
    return codes, alpha, scale


def compress_f64(x, block: int, tau: float = 1.0, eps: float = EPS, fmt: str = "e4m3"):
    """Like compress() for a tensor of float64 values."""
    lib = _load()
    xv = np.ascontiguousarray(x, dtype=np.float64)
    n = xv.size
    if block <= 0 or n % block:
        raise ValueError("element count must be a multiple of the block size")
    codes = np.empty(xv.shape, np.uint8)
    alpha = np.empty(n // block, np.float32)
    scale = np.empty(n // block, np.float32)
    _check(lib.taco_oracle_compress_f64(_ptr(xv), n, block, tau, eps, _fmt(fmt), _ptr(codes),
                                        _ptr(alpha), _ptr(scale)))
    return codes, alpha, scale


def reduce_compress(own_bits, payloads, block: int, tau: float = 1.0, eps: float = EPS,
                    fmt: str = "e4m3"):
    """Owner step: compress own + sum of the payloads' reconstructions.
    own_bits: bf16 bit patterns or None; payloads: list of (codes, alpha, scale)."""
    lib = _load()
    pay = [(np.ascontiguousarray(c, dtype=np.uint8), np.ascontiguousarray(a, dtype=np.float32),
            np.ascontiguousarray(s, dtype=np.float32)) for c, a, s in payloads]
    if own_bits is not None:
        own = np.ascontiguousarray(own_bits, dtype=np.uint16)
        shape, n = own.shape, own.size
    else:
        own = None
        shape, n = pay[0][0].shape, pay[0][0].size
    for c, a, s in pay:
        assert c.size == n and a.size == n // block and s.size == n // block
    arr = ctypes.c_void_p * max(1, len(pay))
    cp = arr(*[c.ctypes.data for c, _, _ in pay])
    ap = arr(*[a.ctypes.data for _, a, _ in pay])
    sp = arr(*[s.ctypes.data for _, _, s in pay])
    codes = np.empty(shape, np.uint8)
    alpha = np.empty(n // block, np.float32)
    scale = np.empty(n // block, np.float32)
    _check(lib.taco_oracle_reduce_compress(None if own is None else _ptr(own), len(pay),
                                           ctypes.cast(cp, ctypes.c_void_p), ctypes.cast(ap, ctypes.c_void_p),
                                           ctypes.cast(sp, ctypes.c_void_p), n, block, tau, eps,
                                           _fmt(fmt), _ptr(codes), _ptr(alpha), _ptr(scale)))
    return codes, alpha, scale


def reconstruct_f64(codes, alpha, scale, block: int, fmt: str = "e4m3") -> np.ndarray:
    """G' in float64 (before any output rounding), same shape as codes."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    out = np.empty(c.shape, np.float64)
    _check(lib.taco_oracle_reconstruct_f64(_ptr(c), _ptr(a), _ptr(s), c.size, block, _fmt(fmt),
                                           _ptr(out)))
    return out


def decompress(codes, alpha, scale, block: int, fmt: str = "e4m3") -> np.ndarray:
    """bf16 bit patterns (uint16) of the reconstruction."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    y = np.empty(c.shape, np.uint16)
    _check(lib.taco_oracle_decompress(_ptr(c), _ptr(a), _ptr(s), c.size, block, _fmt(fmt), _ptr(y)))
    return y


def decompress_accumulate(codes, alpha, scale, block: int, acc: np.ndarray,
                          fmt: str = "e4m3") -> np.ndarray:
    """acc (float32, updated in place and returned) += G'."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    a = np.ascontiguousarray(alpha, dtype=np.float32)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    assert acc.dtype == np.float32 and acc.flags["C_CONTIGUOUS"] and acc.size == c.size
    _check(lib.taco_oracle_decompress_accumulate(_ptr(c), _ptr(a), _ptr(s), c.size, block,
                                                 _fmt(fmt), _ptr(acc)))
    return acc


def decompress_accumulate_n(payloads, block: int, acc: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """acc (float32, updated in place and returned) += the sum of the payloads'
    reconstructions, summed in double and rounded once.  payloads: list of
    (codes, alpha, scale)."""
    lib = _load()
    pay = [(np.ascontiguousarray(c, dtype=np.uint8), np.ascontiguousarray(a, dtype=np.float32),
            np.ascontiguousarray(s, dtype=np.float32)) for c, a, s in payloads]
    assert acc.dtype == np.float32 and acc.flags["C_CONTIGUOUS"]
    n = acc.size
    for c, a, s in pay:
        assert c.size == n and a.size == n // block and s.size == n // block
    arr = ctypes.c_void_p * max(1, len(pay))
    cp = arr(*[c.ctypes.data for c, _, _ in pay])
    ap = arr(*[a.ctypes.data for _, a, _ in pay])
    sp = arr(*[s.ctypes.data for _, _, s in pay])
    _check(lib.taco_oracle_decompress_accumulate_n(len(pay), ctypes.cast(cp, ctypes.c_void_p),
                                                   ctypes.cast(ap, ctypes.c_void_p),
                                                   ctypes.cast(sp, ctypes.c_void_p), n, block,
                                                   _fmt(fmt), _ptr(acc)))
    return acc


def roundtrip_noquant(x_bits, block: int, tau: float = 1.0, eps: float = EPS) -> np.ndarray:
    """Eq. 8 output fed straight to Eq. 12-13 (no quantisation), float64."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    out = np.empty(block, np.float64)
    _check(lib.taco_oracle_roundtrip_noquant(_ptr(x), block, tau, eps, _ptr(out)))
    return out


# ------------------------------------------------- ablation variants ----

#: Round-trip variants (see taco_oracle.c): the operator and the ablations the
#: TACO paper compares it with.
VARIANTS = {"taco": 0, "direct": 1, "ds": 2, "ash": 3, "hadamard": 4, "tensor": 5}


def roundtrip_variant(x_bits, block: int, variant: str, fmt: str = "e4m3", tau: float = 1.0,
                      eps: float = EPS) -> np.ndarray:
    """x' (float64, same shape as x) of one ablation variant's round trip."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r} (one of {sorted(VARIANTS)})")
    out = np.empty(x.shape, np.float64)
    _check(lib.taco_oracle_roundtrip_variant(_ptr(x), x.size, block, VARIANTS[variant], _fmt(fmt),
                                             tau, eps, _ptr(out)))
    return out


def fidelity(ref, got) -> dict:
    """RelL2, Cos, MaxErr and MSE of got against ref (GIFT Eq. 21), in double."""
    lib = _load()
    r = np.ascontiguousarray(ref, dtype=np.float64).reshape(-1)
    g = np.ascontiguousarray(got, dtype=np.float64).reshape(-1)
    assert r.size == g.size and r.size > 0
    out = np.empty(4, np.float64)
    _check(lib.taco_oracle_fidelity(_ptr(r), _ptr(g), r.size, _ptr(out)))
    return {"rel_l2": float(out[0]), "cos": float(out[1]), "max_err": float(out[2]),
            "mse": float(out[3])}


# ---------------------------------------------------- wire layout -------

def pack(codes, alpha, scale, block: int) -> np.ndarray:
    """Interleaved wire layout of TACO section 4.4.2 (alpha_k and s_k stored
    contiguously with block k's FP8 payload): one record of block + 8 bytes
    per block, the block's codes followed by alpha_k and s_k as
    little-endian float32 (Algorithm 1 communicates the tuple in the order
    (q_k, alpha_k, s_k)).  Returns uint8 [M, block + 8]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    a = np.ascontiguousarray(alpha, dtype='<f4').reshape(-1)
    s = np.ascontiguousarray(scale, dtype='<f4').reshape(-1)
    m = a.size
    assert c.size == m * block and s.size == m
    out = np.empty((m, block + 8), np.uint8)
    out[:, :block] = c.reshape(m, block)
    out[:, block:block + 4] = a.view(np.uint8).reshape(m, 4)
    out[:, block + 4:] = s.view(np.uint8).reshape(m, 4)
    return out


def unpack(payload, block: int):
    """(codes [M*block], alpha [M], scale [M]) of an interleaved payload."""
    p = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1, block + 8)
    codes = p[:, :block].reshape(-1).copy()
    alpha = p[:, block:block + 4].copy().view('<f4').reshape(-1).astype(np.float32)
    scale = p[:, block + 4:].copy().view('<f4').reshape(-1).astype(np.float32)
    return codes, alpha, scale


# ------------------------------------------------------------ helpers ----

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
