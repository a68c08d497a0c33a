"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects every bad argument before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

# These tests pass fake device addresses and only ever expect validation
# errors; on a machine with a GPU a validation slip would launch a kernel on
# them, so the module runs only where no GPU is visible (counting devices
# does not initialise the GPU).
try:
    import torch as _torch
    if _torch.cuda.device_count() > 0:
        pytest.skip("host-only validation tests (fake device pointers)", allow_module_level=True)
except ImportError:  # pragma: no cover
    pass

HEADER = os.path.join(ROOT, "include", "taco.h")
LIB = os.path.join(ROOT, "gradients_taco_compress_amd", "libtaco.so")

OK, NULL, SHAPE, BLOCK, PARAM, ALIGN, ALIAS, HIP, FORMAT = range(9)
E4M3, E5M2, INT8 = range(3)
A = 1 << 20          # fake, 16-byte aligned "device" addresses: never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(taco_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libtaco.so is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.taco_num_blocks.argtypes = [I64, I64, I32]
    L.taco_num_blocks.restype = I64
    L.taco_compress.argtypes = [P, I64, I64, I32, F32, P, P, P, P]
    L.taco_decompress.argtypes = [P, P, P, I64, I64, I32, P, P]
    L.taco_decompress_accumulate.argtypes = [P, P, P, I64, I64, I32, P, P]
    L.taco_reduce_compress.argtypes = [P, I32, P, P, P, I64, I64, I32, F32, P, P, P, P]
    L.taco_packed_bytes.argtypes = [I64, I64, I32]
    L.taco_packed_bytes.restype = I64
    L.taco_compress_packed.argtypes = [P, I64, I64, I32, F32, P, P]
    L.taco_decompress_packed.argtypes = [P, I64, I64, I32, P, P]
    L.taco_decompress_accumulate_packed.argtypes = [P, I64, I64, I32, P, P]
    L.taco_reduce_compress_packed.argtypes = [P, I32, P, I64, I64, I32, F32, P, P]
    L.taco_e4m3_encode.argtypes = [P, I64, P, P]
    L.taco_e4m3_decode.argtypes = [P, I64, P, P]
    L.taco_compress_fmt.argtypes = [P, I64, I64, I32, F32, I32, P, P, P, P]
    L.taco_decompress_fmt.argtypes = [P, P, P, I64, I64, I32, I32, P, P]
    L.taco_decompress_accumulate_fmt.argtypes = [P, P, P, I64, I64, I32, I32, P, P]
    L.taco_reduce_compress_fmt.argtypes = [P, I32, P, P, P, I64, I64, I32, F32, I32, P, P, P, P]
    L.taco_compress_packed_fmt.argtypes = [P, I64, I64, I32, F32, I32, P, P]
    L.taco_decompress_packed_fmt.argtypes = [P, I64, I64, I32, I32, P, P]
    L.taco_decompress_accumulate_packed_fmt.argtypes = [P, I64, I64, I32, I32, P, P]
    L.taco_reduce_compress_packed_fmt.argtypes = [P, I32, P, I64, I64, I32, F32, I32, P, P]
    L.taco_roundtrip.argtypes = [P, I64, I64, I32, F32, I32, I32, P, P, P]
    L.taco_roundtrip_noalloc.argtypes = [P, I64, I64, I32, F32, I32, I32, P, P, P]
    L.taco_decompress_accumulate_n.argtypes = [I32, P, P, P, I64, I64, I32, P, P]
    L.taco_decompress_accumulate_n_fmt.argtypes = [I32, P, P, P, I64, I64, I32, I32, P, P]
    L.taco_decompress_accumulate_n_packed.argtypes = [I32, P, I64, I64, I32, P, P]
    L.taco_decompress_accumulate_n_packed_fmt.argtypes = [I32, P, I64, I64, I32, I32, P, P]
    L.taco_encode.argtypes = [I32, P, I64, P, P]
    L.taco_decode.argtypes = [I32, P, I64, P, P]
    L.taco_status_string.argtypes = [ctypes.c_int]
    L.taco_status_string.restype = ctypes.c_char_p
    return L


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) == 29, names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (taco_\w+)", out))
    assert exported == set(names), exported ^ set(names)


def test_binding_names_match_header():
    import importlib.util
    spec = importlib.util.find_spec("gradients_taco_compress_amd")
    assert spec is not None
    import gradients_taco_compress_amd as taco
    assert set(taco.EXPORTS) == set(declared_functions())
    for n in declared_functions():
        assert callable(getattr(taco, n))


def test_status_strings(lib):
    for s in range(9):
        assert lib.taco_status_string(s)
    assert b"format" in lib.taco_status_string(FORMAT)
    assert lib.taco_status_string(99) == b"unknown status"


def test_num_blocks(lib):
    assert lib.taco_num_blocks(8192, 2560, 128) == 8192 * 2560 // 128
    assert lib.taco_num_blocks(0, 1024, 256) == 0
    assert lib.taco_num_blocks(3, 96, 128) == -1          # 288 % 128 != 0
    assert lib.taco_num_blocks(4, 96, 128) == 3          # blocks may cross rows
    assert lib.taco_num_blocks(-1, 128, 128) == -1
    assert lib.taco_num_blocks(1, 0, 128) == -1
    assert lib.taco_num_blocks(1, 1024, 100) == -1
    assert lib.taco_num_blocks(1 << 40, 1 << 40, 128) == -1   # overflow


def compress(lib, x=A, tokens=4, hidden=256, block=128, tau=1.0,
             codes=2 * A, alpha=3 * A, scale=4 * A):
    return lib.taco_compress(x, tokens, hidden, block, tau, codes, alpha, scale, None)


def test_compress_validation(lib):
    assert compress(lib, tokens=-1) == SHAPE
    assert compress(lib, hidden=0) == SHAPE
    assert compress(lib, tokens=3, hidden=96) == SHAPE
    assert compress(lib, tokens=1 << 40, hidden=1 << 40) == SHAPE
    for b in (0, 16, 100, 1024, -128):
        assert compress(lib, block=b) == BLOCK
    for tau in (0.0, -1.0, float("inf"), float("nan"), 1e21):
        assert compress(lib, tau=tau) == PARAM
    assert compress(lib, x=None) == NULL
    assert compress(lib, codes=None) == NULL
    assert compress(lib, alpha=None) == NULL
    assert compress(lib, scale=None) == NULL
    assert compress(lib, x=A + 8) == ALIGN
    assert compress(lib, codes=2 * A + 4) == ALIGN
    assert compress(lib, alpha=3 * A + 2) == ALIGN
    # Outputs overlapping the input or each other.
    assert compress(lib, codes=A + 1024) == ALIAS
    assert compress(lib, alpha=A + 16) == ALIAS
    assert compress(lib, scale=3 * A + 4) == ALIAS
    assert compress(lib, codes=3 * A - 512) == ALIAS
    # Empty tensors are a no-op, even with NULL pointers.
    assert compress(lib, tokens=0, x=None, codes=None, alpha=None, scale=None) == OK


def receiver(fn, lib, codes=A, alpha=2 * A, scale=3 * A, tokens=4, hidden=256, block=128,
             out=4 * A):
    return fn(codes, alpha, scale, tokens, hidden, block, out, None)


@pytest.mark.parametrize("name,elem", [("taco_decompress", 2), ("taco_decompress_accumulate", 4)])
def test_receiver_validation(lib, name, elem):
    fn = getattr(lib, name)
    assert receiver(fn, lib, tokens=-2) == SHAPE
    assert receiver(fn, lib, tokens=3, hidden=96) == SHAPE
    assert receiver(fn, lib, block=48) == BLOCK
    assert receiver(fn, lib, codes=None) == NULL
    assert receiver(fn, lib, alpha=None) == NULL
    assert receiver(fn, lib, scale=None) == NULL
    assert receiver(fn, lib, out=None) == NULL
    assert receiver(fn, lib, out=4 * A + 8) == ALIGN
    assert receiver(fn, lib, codes=A + 8) == ALIGN
    assert receiver(fn, lib, scale=3 * A + 1) == ALIGN
    assert receiver(fn, lib, out=A + 512) == ALIAS
    assert receiver(fn, lib, out=2 * A - 16) == ALIAS
    assert receiver(fn, lib, scale=4 * A + 4 * 256 * elem - 4) == ALIAS
    assert receiver(fn, lib, tokens=0, codes=None, alpha=None, scale=None, out=None) == OK


def test_codec_validation(lib):
    assert lib.taco_e4m3_encode(A, -1, 2 * A, None) == SHAPE
    assert lib.taco_e4m3_encode(A, 0, None, None) == OK
    assert lib.taco_e4m3_encode(None, 16, 2 * A, None) == NULL
    assert lib.taco_e4m3_encode(A + 4, 16, 2 * A, None) == ALIGN
    assert lib.taco_e4m3_encode(A, 16, A + 32, None) == ALIAS
    assert lib.taco_e4m3_decode(A, 16, None, None) == NULL
    assert lib.taco_e4m3_decode(A, 16, A, None) == ALIAS
    assert lib.taco_e4m3_decode(A + 1, 16, 2 * A, None) == ALIGN


def reduce_call(lib, own=A, npay=2, codes=(5 * A, 6 * A), alpha=(7 * A, 8 * A),
                scale=(9 * A, 10 * A), tokens=4, hidden=256, block=128, tau=1.0,
                out_codes=2 * A, out_alpha=3 * A, out_scale=4 * A):
    arr = ctypes.c_void_p * 8
    c = None if codes is None else ctypes.cast(arr(*codes), ctypes.c_void_p)
    a = None if alpha is None else ctypes.cast(arr(*alpha), ctypes.c_void_p)
    s = None if scale is None else ctypes.cast(arr(*scale), ctypes.c_void_p)
    return lib.taco_reduce_compress(own, npay, c, a, s, tokens, hidden, block, tau,
                                    out_codes, out_alpha, out_scale, None)


def test_reduce_compress_validation(lib):
    assert reduce_call(lib, tokens=-1) == SHAPE
    assert reduce_call(lib, tokens=3, hidden=96) == SHAPE
    assert reduce_call(lib, block=96) == BLOCK
    assert reduce_call(lib, tau=0.0) == PARAM
    assert reduce_call(lib, npay=9) == PARAM
    assert reduce_call(lib, npay=-1) == PARAM
    assert reduce_call(lib, own=None, npay=0) == PARAM
    assert reduce_call(lib, out_codes=None) == NULL
    assert reduce_call(lib, codes=None) == NULL
    assert reduce_call(lib, codes=(5 * A, None)) == NULL
    assert reduce_call(lib, own=A + 8) == ALIGN
    assert reduce_call(lib, codes=(5 * A, 6 * A + 4)) == ALIGN
    assert reduce_call(lib, scale=(9 * A + 2, 10 * A)) == ALIGN
    assert reduce_call(lib, out_codes=A + 256) == ALIAS          # overlaps own
    assert reduce_call(lib, out_alpha=5 * A + 64) == ALIAS       # overlaps payload 0 codes
    assert reduce_call(lib, out_scale=8 * A) == ALIAS            # overlaps payload 1 alpha
    assert reduce_call(lib, out_scale=3 * A + 4) == ALIAS        # overlaps out_alpha
    # Empty tensors: a no-op once the arguments that do not depend on N are valid.
    assert reduce_call(lib, tokens=0, out_codes=None, out_alpha=None, out_scale=None) == OK
    assert reduce_call(lib, own=None, npay=1, tokens=0) == OK   # own is optional


def test_packed_validation(lib):
    assert lib.taco_packed_bytes(4, 256, 128) == 8 * 136
    assert lib.taco_packed_bytes(3, 96, 128) == -1
    assert lib.taco_packed_bytes(4, 256, 100) == -1
    cp = lambda **k: lib.taco_compress_packed(k.get("x", A), k.get("tokens", 4), 256,
                                              k.get("block", 128), k.get("tau", 1.0),
                                              k.get("out", 2 * A), None)
    assert cp(tokens=-1) == SHAPE
    assert cp(block=48) == BLOCK
    assert cp(tau=-1.0) == PARAM
    assert cp(x=None) == NULL
    assert cp(out=None) == NULL
    assert cp(out=2 * A + 8) == ALIGN
    assert cp(out=A + 1024) == ALIAS
    assert cp(tokens=0, x=None, out=None) == OK
    for fn, elem in ((lib.taco_decompress_packed, 2), (lib.taco_decompress_accumulate_packed, 4)):
        dp = lambda **k: fn(k.get("pay", A), k.get("tokens", 4), 256, k.get("block", 128),
                            k.get("out", 2 * A), None)
        assert dp(tokens=-3) == SHAPE
        assert dp(block=96) == BLOCK
        assert dp(pay=None) == NULL
        assert dp(out=None) == NULL
        assert dp(pay=A + 4) == ALIGN
        assert dp(out=A + 8 * 136 - 16) == ALIAS
        assert dp(tokens=0, pay=None, out=None) == OK
    arr = ctypes.c_void_p * 8
    rp = lambda own=A, npay=2, pays=(5 * A, 6 * A), out=2 * A, tokens=4: lib.taco_reduce_compress_packed(
        own, npay, None if pays is None else ctypes.cast(arr(*pays), ctypes.c_void_p), tokens, 256,
        128, 1.0, out, None)
    assert rp(npay=9) == PARAM
    assert rp(own=None, npay=0) == PARAM
    assert rp(out=None) == NULL
    assert rp(pays=None) == NULL
    assert rp(pays=(5 * A, None)) == NULL
    assert rp(pays=(5 * A, 6 * A + 8)) == ALIGN
    assert rp(out=5 * A + 512) == ALIAS
    assert rp(out=A + 64) == ALIAS
    assert rp(tokens=0, out=None) == OK


def test_format_validation(lib):
    """A bad format is reported first (also for an empty tensor); with a
    valid format every other check is the same as without one."""
    arr = ctypes.c_void_p * 8
    pays = ctypes.cast(arr(5 * A, 6 * A), ctypes.c_void_p)
    calls = {
        "compress": lambda f, **k: lib.taco_compress_fmt(
            k.get("x", A), k.get("tokens", 4), 256, 128, 1.0, f, 2 * A, 3 * A, 4 * A, None),
        "decompress": lambda f, **k: lib.taco_decompress_fmt(
            k.get("x", A), 2 * A, 3 * A, k.get("tokens", 4), 256, 128, f, 4 * A, None),
        "accumulate": lambda f, **k: lib.taco_decompress_accumulate_fmt(
            k.get("x", A), 2 * A, 3 * A, k.get("tokens", 4), 256, 128, f, 4 * A, None),
        # (own is optional: the probed pointer is the required output)
        "reduce": lambda f, **k: lib.taco_reduce_compress_fmt(
            A, 2, pays, pays, pays, k.get("tokens", 4), 256, 128, 1.0, f,
            k.get("x", 2 * A), 3 * A, 4 * A, None),
        "compress_packed": lambda f, **k: lib.taco_compress_packed_fmt(
            k.get("x", A), k.get("tokens", 4), 256, 128, 1.0, f, 2 * A, None),
        "decompress_packed": lambda f, **k: lib.taco_decompress_packed_fmt(
            k.get("x", A), k.get("tokens", 4), 256, 128, f, 2 * A, None),
        "accumulate_packed": lambda f, **k: lib.taco_decompress_accumulate_packed_fmt(
            k.get("x", A), k.get("tokens", 4), 256, 128, f, 2 * A, None),
        "reduce_packed": lambda f, **k: lib.taco_reduce_compress_packed_fmt(
            A, 2, pays, k.get("tokens", 4), 256, 128, 1.0, f, k.get("x", 2 * A), None),
        "encode": lambda f, **k: lib.taco_encode(f, k.get("x", A), 16 if k.get("tokens", 4)
                                                 else 0, 2 * A, None),
        "decode": lambda f, **k: lib.taco_decode(f, k.get("x", A), 16 if k.get("tokens", 4)
                                                 else 0, 2 * A, None),
    }
    for name, call in calls.items():
        for bad in (-1, 3, 255):
            assert call(bad) == FORMAT, name
            assert call(bad, tokens=0) == FORMAT, name
        for f in (E4M3, E5M2, INT8):
            assert call(f, x=None) == NULL, (name, f)
            assert call(f, x=9 * A + 2) == ALIGN, (name, f)
            assert call(f, tokens=0, x=None) == OK, (name, f)
            if name not in ("encode", "decode"):
                assert call(f, tokens=-1) == SHAPE, (name, f)


def test_format_calls_match_e4m3_calls_on_errors(lib):
    """The calls without a format behave as the E4M3 calls with one."""
    # (only argument sets that fail validation: the pointers are fake)
    for hidden, block, tau, want in ((96, 128, 1.0, SHAPE), (256, 100, 1.0, BLOCK),
                                     (256, 128, -1.0, PARAM)):
        a = lib.taco_compress(A, 3, hidden, block, tau, 2 * A, 3 * A, 4 * A, None)
        b = lib.taco_compress_fmt(A, 3, hidden, block, tau, E4M3, 2 * A, 3 * A, 4 * A, None)
        assert a == b == want


def test_roundtrip_validation(lib):
    rt = lambda **k: lib.taco_roundtrip(k.get("x", A), k.get("tokens", 4), k.get("hidden", 256),
                                        k.get("block", 128), k.get("tau", 1.0),
                                        k.get("fmt", E4M3), k.get("variant", 0),
                                        k.get("y", 2 * A), k.get("sums", 3 * A), None)
    assert rt(fmt=7) == FORMAT
    assert rt(fmt=7, tokens=0) == FORMAT
    assert rt(tokens=-1) == SHAPE
    assert rt(hidden=96, tokens=3) == SHAPE
    assert rt(block=48) == BLOCK
    assert rt(tau=0.0) == PARAM
    for bad in (-1, 6, 99):
        assert rt(variant=bad) == PARAM
    assert rt(sums=None) == NULL
    assert rt(x=None) == NULL
    assert rt(sums=3 * A + 4) == ALIGN
    assert rt(x=A + 8) == ALIGN
    assert rt(y=2 * A + 2) == ALIGN
    assert rt(sums=A + 64) == ALIAS            # inside x
    assert rt(sums=2 * A + 512) == ALIAS       # inside y
    assert rt(y=A + 1024) == ALIAS             # y overlaps x
    assert rt(tokens=0, x=None, y=None, sums=None) == OK   # empty: nothing written


def test_roundtrip_noalloc_validation(lib):
    """The no-allocation round trip validates like taco_roundtrip, with the
    40-byte totals in place of the sums; an argument set that passes every
    check reaches the device lookup, which fails without a GPU."""
    rt = lambda **k: lib.taco_roundtrip_noalloc(
        k.get("x", A), k.get("tokens", 4), k.get("hidden", 256), k.get("block", 128),
        k.get("tau", 1.0), k.get("fmt", E4M3), k.get("variant", 0), k.get("y", 2 * A),
        k.get("totals", 3 * A), None)
    assert rt(fmt=7) == FORMAT
    assert rt(fmt=7, tokens=0) == FORMAT
    assert rt(tokens=-1) == SHAPE
    assert rt(hidden=96, tokens=3) == SHAPE
    assert rt(block=48) == BLOCK
    assert rt(tau=0.0) == PARAM and rt(tau=float("nan")) == PARAM
    for bad in (-1, 6, 99):
        assert rt(variant=bad) == PARAM
    assert rt(totals=None) == NULL
    assert rt(x=None) == NULL
    assert rt(totals=3 * A + 4) == ALIGN
    assert rt(x=A + 8) == ALIGN
    assert rt(y=2 * A + 2) == ALIGN
    assert rt(totals=A + 64) == ALIAS            # inside x
    assert rt(totals=2 * A + 512) == ALIAS       # inside y
    assert rt(totals=2 * A - 32) == ALIAS        # its 40 bytes reach into y
    assert rt(y=A + 1024) == ALIAS               # y overlaps x
    assert rt(tokens=0, x=None, y=None, totals=None) == OK   # empty: nothing written
    # Every check passes: the device lookup (no GPU here) refuses the launch.
    assert rt(totals=2 * A - 40) == HIP          # ends right where y starts
    assert rt(y=None) == HIP


def test_accumulate_n_validation(lib):
    arr = ctypes.c_void_p * 8
    cs = lambda *v: None if v == (None,) else ctypes.cast(arr(*v), ctypes.c_void_p)
    an = lambda **k: lib.taco_decompress_accumulate_n(
        k.get("npay", 2), k.get("codes", cs(5 * A, 6 * A)), k.get("alpha", cs(7 * A, 8 * A)),
        k.get("scale", cs(9 * A, 10 * A)), k.get("tokens", 4), k.get("hidden", 256),
        k.get("block", 128), k.get("acc", 2 * A), None)
    assert an(tokens=-1) == SHAPE
    assert an(hidden=96, tokens=3) == SHAPE
    assert an(block=48) == BLOCK
    assert an(npay=9) == PARAM and an(npay=-1) == PARAM
    assert an(acc=None) == NULL
    assert an(codes=None) == NULL
    assert an(codes=cs(5 * A, None)) == NULL
    assert an(acc=2 * A + 8) == ALIGN
    assert an(codes=cs(5 * A, 6 * A + 4)) == ALIGN
    assert an(acc=5 * A - 64) == ALIAS          # acc overlaps payload 0's codes
    assert an(acc=9 * A - 1024) == ALIAS        # acc overlaps payload 0's scale
    # Nothing to do: empty tensors and zero payloads, even with NULL pointers.
    assert an(tokens=0, acc=None, codes=None, alpha=None, scale=None) == OK
    assert an(npay=0, acc=None, codes=None, alpha=None, scale=None) == OK
    assert lib.taco_decompress_accumulate_n_fmt(2, None, None, None, 4, 256, 128, 9, 2 * A,
                                                None) == FORMAT
    ap = lambda **k: lib.taco_decompress_accumulate_n_packed(
        k.get("npay", 2), k.get("pays", cs(5 * A, 6 * A)), 4, 256, 128, k.get("acc", 2 * A), None)
    assert ap(pays=None) == NULL
    assert ap(pays=cs(5 * A, 6 * A + 8)) == ALIGN
    assert ap(acc=5 * A + 64) == ALIAS
    assert ap(npay=0, pays=None, acc=None) == OK
    assert lib.taco_decompress_accumulate_n_packed_fmt(2, None, 4, 256, 128, 3, 2 * A,
                                                       None) == FORMAT


PROBE_HEADER = os.path.join(ROOT, "include", "taco_probe.h")
PROBE_LIB = os.path.join(ROOT, "gradients_taco_compress_amd", "libtaco_probe.so")


def test_probe_library_exports_and_validation():
    """The measurement library exports exactly what its header declares and
    refuses bad arguments before any launch (without a GPU a valid call
    fails at the launch)."""
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(taco_probe_[a-z0-9_]+)\s*\(", text)))
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True,
                         text=True).stdout
    assert set(re.findall(r" T (taco_\w+)", out)) == set(names) == {"taco_probe_empty",
                                                                    "taco_probe_stream"}
    import gradients_taco_compress_amd.probe as probe
    assert set(probe.EXPORTS) == set(names)
    L = ctypes.CDLL(PROBE_LIB)
    L.taco_probe_empty.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    L.taco_probe_stream.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]
    ARGS, LAUNCH = 1, 2
    assert L.taco_probe_empty(0, None) == ARGS
    assert L.taco_probe_empty(1 << 24, None) == ARGS          # 2^32 threads: too many
    assert L.taco_probe_empty(5120, None) == LAUNCH
    st = lambda ld=2, sto=1, src=A, dst=64 * A, waves=1024, valu=0: L.taco_probe_stream(
        ld, sto, valu, src, dst, waves, None)
    assert st(ld=3) == ARGS and st(ld=2, sto=2) == ARGS        # unsupported mixes
    assert st(waves=0) == ARGS
    assert st(valu=-4) == ARGS and st(valu=6) == ARGS and st(valu=1 << 20) == ARGS
    assert st(valu=276) == LAUNCH
    assert st(src=None) == ARGS and st(dst=A + 8) == ARGS     # null, misaligned
    assert st(dst=A + 1024) == ARGS                            # overlap
    assert st(dst=A + 2 * 1024 * 1024) == LAUNCH               # just past src
    for ld, sto in probe.MIXES.values():
        assert st(ld=ld, sto=sto) == LAUNCH
