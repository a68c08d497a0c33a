"""Seeded random argument sets against the C ABI's validation, without a GPU.

An independent model of the rules include/taco.h states (checked in order:
format, shape, block, divisibility, target energy, empty tensor, null
pointers, alignment, overlap) predicts each call's status; a call that passes
every check reaches the launch, which on a machine without a GPU fails with
TACO_ERR_HIP.  So every status the library returns is compared with the
model's, for compress, decompress, accumulate and both interleaved calls, in
both the E4M3 and the format-taking forms.
"""
import ctypes
import os

import numpy as np
import pytest

from conftest import ROOT

# Fake device addresses: the module must never run where a launch could
# reach a GPU (counting devices does not initialise one).
try:
    import torch as _torch
    if _torch.cuda.device_count() > 0:
        pytest.skip("host-only validation fuzz (fake device pointers)", allow_module_level=True)
except ImportError:  # pragma: no cover
    pass

OK, NULL, SHAPE, BLOCK, PARAM, ALIGN, ALIAS, HIP, FORMAT = range(9)
LIB = os.path.join(ROOT, "gradients_taco_compress_amd", "libtaco.so")
BLOCKS = (32, 64, 128, 256, 512)
MAX_TAU = np.float32(1e20)


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.taco_compress.argtypes = [P, I64, I64, I32, F32, P, P, P, P]
    L.taco_compress_fmt.argtypes = [P, I64, I64, I32, F32, I32, P, P, P, P]
    L.taco_decompress.argtypes = [P, P, P, I64, I64, I32, P, P]
    L.taco_decompress_fmt.argtypes = [P, P, P, I64, I64, I32, I32, P, P]
    L.taco_decompress_accumulate.argtypes = [P, P, P, I64, I64, I32, P, P]
    L.taco_decompress_accumulate_fmt.argtypes = [P, P, P, I64, I64, I32, I32, P, P]
    L.taco_compress_packed_fmt.argtypes = [P, I64, I64, I32, F32, I32, P, P]
    L.taco_decompress_packed_fmt.argtypes = [P, I64, I64, I32, I32, P, P]
    L.taco_decompress_accumulate_packed_fmt.argtypes = [P, I64, I64, I32, I32, P, P]
    return L


# ------------------------------------------------------------ the model --

def _numel(tokens, hidden):
    if tokens < 0 or hidden <= 0:
        return None
    if tokens > 0 and hidden > (1 << 60) // tokens:
        return None
    return tokens * hidden


def _shape(tokens, hidden, block):
    """(status or None, n)."""
    n = _numel(tokens, hidden)
    if n is None:
        return SHAPE, 0
    if block not in BLOCKS:
        return BLOCK, 0
    if n % block:
        return SHAPE, 0
    return None, n


def _overlap(a, na, b, nb):
    return na > 0 and nb > 0 and a < b + nb and b < a + na


def _tau_ok(tau):
    t = np.float32(tau)
    return bool(t > 0) and bool(t <= MAX_TAU)


def model_compress(fmt, x, tokens, hidden, block, tau, codes, alpha, scale):
    if fmt not in (0, 1, 2):
        return FORMAT
    st, n = _shape(tokens, hidden, block)
    if st is not None:
        return st
    if not _tau_ok(tau):
        return PARAM
    if n == 0:
        return OK
    if 0 in (x, codes, alpha, scale):
        return NULL
    if x % 16 or codes % 16 or alpha % 4 or scale % 4:
        return ALIGN
    m = n // block
    bufs = [(codes, n), (alpha, 4 * m), (scale, 4 * m)]
    for i, (p, np_) in enumerate(bufs):
        if _overlap(p, np_, x, 2 * n):
            return ALIAS
        for q, nq in bufs[i + 1:]:
            if _overlap(p, np_, q, nq):
                return ALIAS
    return HIP


def model_receive(fmt, codes, alpha, scale, tokens, hidden, block, out, elem):
    if fmt not in (0, 1, 2):
        return FORMAT
    st, n = _shape(tokens, hidden, block)
    if st is not None:
        return st
    if n == 0:
        return OK
    if 0 in (codes, alpha, scale, out):
        return NULL
    if codes % 16 or out % 16 or alpha % 4 or scale % 4:
        return ALIGN
    m = n // block
    for p, np_ in ((codes, n), (alpha, 4 * m), (scale, 4 * m)):
        if _overlap(out, elem * n, p, np_):
            return ALIAS
    return HIP


def model_compress_packed(fmt, x, tokens, hidden, block, tau, payload):
    if fmt not in (0, 1, 2):
        return FORMAT
    st, n = _shape(tokens, hidden, block)
    if st is not None:
        return st
    if not _tau_ok(tau):
        return PARAM
    if n == 0:
        return OK
    if 0 in (x, payload):
        return NULL
    if x % 16 or payload % 16:
        return ALIGN
    if _overlap(payload, (n // block) * (block + 8), x, 2 * n):
        return ALIAS
    return HIP


def model_receive_packed(fmt, payload, tokens, hidden, block, out, elem):
    if fmt not in (0, 1, 2):
        return FORMAT
    st, n = _shape(tokens, hidden, block)
    if st is not None:
        return st
    if n == 0:
        return OK
    if 0 in (payload, out):
        return NULL
    if payload % 16 or out % 16:
        return ALIGN
    if _overlap(out, elem * n, payload, (n // block) * (block + 8)):
        return ALIAS
    return HIP


# ------------------------------------------------------- the generator --

class Gen:
    """Argument sets biased towards the deep checks: most shapes are valid,
    pointers are laid out disjoint and then perturbed (null, misaligned,
    moved into another buffer)."""

    def __init__(self, seed):
        self.r = np.random.default_rng(seed)

    def pick(self, seq):
        return seq[int(self.r.integers(len(seq)))]

    def shape(self):
        r = self.r
        if r.random() < 0.75:
            block = self.pick(BLOCKS)
            hidden = block * int(r.integers(1, 9)) if r.random() < 0.8 else int(r.integers(1, 5)) * 64
            tokens = int(r.integers(0, 40))
        else:
            tokens = self.pick([-1, 0, 1, 3, 1 << 20, 1 << 40, (1 << 62) + 1])
            hidden = self.pick([-7, 0, 1, 31, 96, 128, 4096, 1 << 30, 1 << 60])
            block = self.pick([-128, 0, 16, 48, 32, 64, 128, 256, 512, 1024])
        return tokens, hidden, block

    def tau(self):
        if self.r.random() < 0.85:
            return 1.0
        return self.pick([0.0, -1.0, float("nan"), float("inf"), 1e20, 1.0000001e20, 1e21,
                          1e-30, 3.0e38, 37.5])

    def fmt(self):
        return 0 if self.r.random() < 0.9 else self.pick([-1, 3, 7, 1, 2])

    def pointers(self, sizes):
        """Disjoint 256-aligned buffers of the given byte sizes, then at most
        two perturbations."""
        r = self.r
        ptrs, cur = [], 1 << 24
        for s in sizes:
            ptrs.append(cur)
            cur += ((max(int(s), 1) + 255) // 256) * 256 + 256 * int(r.integers(0, 3))
        for _ in range(int(r.integers(0, 3))):
            i = int(r.integers(len(ptrs)))
            kind = r.random()
            if kind < 0.25:
                ptrs[i] = 0
            elif kind < 0.55:
                ptrs[i] += int(r.integers(1, 16))
            else:                                     # into (or just past) another buffer
                j = int(r.integers(len(ptrs)))
                if ptrs[j]:
                    off = int(r.integers(0, max(1, int(sizes[j]) + 64)))
                    ptrs[i] = ptrs[j] + (off // 16) * 16
        return ptrs


def _sizes(tokens, hidden, block):
    n = _numel(tokens, hidden) or 0
    n = min(n, 1 << 40)
    m = n // block if block > 0 else 0
    return n, m


CASES = 4000


def test_compress_matches_model(lib):
    g = Gen(1)
    seen = set()
    for _ in range(CASES):
        tokens, hidden, block = g.shape()
        tau, fmt = g.tau(), g.fmt()
        n, m = _sizes(tokens, hidden, block)
        x, codes, alpha, scale = g.pointers([2 * n, n, 4 * m, 4 * m])
        want = model_compress(fmt, x, tokens, hidden, block, tau, codes, alpha, scale)
        if fmt == 0:
            got = lib.taco_compress(x, tokens, hidden, block, tau, codes, alpha, scale, None)
            assert got == want, (tokens, hidden, block, tau, x, codes, alpha, scale)
        got = lib.taco_compress_fmt(x, tokens, hidden, block, tau, fmt, codes, alpha, scale, None)
        assert got == want, (fmt, tokens, hidden, block, tau, x, codes, alpha, scale)
        seen.add(want)
    assert seen == {OK, NULL, SHAPE, BLOCK, PARAM, ALIGN, ALIAS, HIP, FORMAT}


@pytest.mark.parametrize("accumulate", [False, True])
def test_receive_matches_model(lib, accumulate):
    g = Gen(2 + accumulate)
    elem = 4 if accumulate else 2
    plain = lib.taco_decompress_accumulate if accumulate else lib.taco_decompress
    withfmt = lib.taco_decompress_accumulate_fmt if accumulate else lib.taco_decompress_fmt
    seen = set()
    for _ in range(CASES):
        tokens, hidden, block = g.shape()
        fmt = g.fmt()
        n, m = _sizes(tokens, hidden, block)
        codes, alpha, scale, out = g.pointers([n, 4 * m, 4 * m, elem * n])
        want = model_receive(fmt, codes, alpha, scale, tokens, hidden, block, out, elem)
        if fmt == 0:
            assert plain(codes, alpha, scale, tokens, hidden, block, out, None) == want
        got = withfmt(codes, alpha, scale, tokens, hidden, block, fmt, out, None)
        assert got == want, (fmt, tokens, hidden, block, codes, alpha, scale, out)
        seen.add(want)
    assert seen == {OK, NULL, SHAPE, BLOCK, ALIGN, ALIAS, HIP, FORMAT}


def test_packed_calls_match_model(lib):
    g = Gen(4)
    seen = set()
    for i in range(CASES):
        tokens, hidden, block = g.shape()
        fmt = g.fmt()
        n, m = _sizes(tokens, hidden, block)
        rec = m * (block + 8) if block > 0 else 0
        if i % 3 == 0:
            tau = g.tau()
            x, payload = g.pointers([2 * n, rec])
            want = model_compress_packed(fmt, x, tokens, hidden, block, tau, payload)
            got = lib.taco_compress_packed_fmt(x, tokens, hidden, block, tau, fmt, payload, None)
        else:
            elem = 2 if i % 3 == 1 else 4
            payload, out = g.pointers([rec, elem * n])
            want = model_receive_packed(fmt, payload, tokens, hidden, block, out, elem)
            fn = (lib.taco_decompress_packed_fmt if elem == 2
                  else lib.taco_decompress_accumulate_packed_fmt)
            got = fn(payload, tokens, hidden, block, fmt, out, None)
        assert got == want, (i, fmt, tokens, hidden, block)
        seen.add(want)
    assert seen == {OK, NULL, SHAPE, BLOCK, PARAM, ALIGN, ALIAS, HIP, FORMAT}
