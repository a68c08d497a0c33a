"""Shared fixtures.  Tests marked ``gpu`` need an MI355X; everything else runs on
the CPU (oracle pins, host-side validation, symbol checks)."""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HELPERS = os.path.join(ROOT, "tests", "helpers")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")


# The code-flip rate is asserted on the totals of the whole session, after
# every test file has run: each comparison of codes against the oracle adds
# its flips and elements to tests/parity.py's TOTALS (per kind and format).
_FLIP_REPORT = []


def pytest_sessionfinish(session, exitstatus):
    parity = sys.modules.get("parity")
    if parity is None:
        return
    lines, ok = parity.session_check()
    _FLIP_REPORT[:] = lines
    if not ok and session.exitstatus == 0:
        session.exitstatus = pytest.ExitCode.TESTS_FAILED


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    for line in _FLIP_REPORT:
        terminalreporter.write_line(line)


def build_helper(name: str) -> str:
    """Compile tests/helpers/<name>.c into a shared library next to it."""
    src = os.path.join(HELPERS, name + ".c")
    lib = os.path.join(HELPERS, "lib" + name + ".so")
    if not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
        tmp = lib + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, lib)
    return lib


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def synth_mod():
    import synth
    synth.build()
    return synth


def read_golden(name: str):
    """Rows of a whitespace-separated fixture, comments (#) stripped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def cpu_threads() -> int:
    try:
        return max(1, min(len(os.sched_getaffinity(0)), 16))
    except AttributeError:  # pragma: no cover
        return 1


def torch_e4m3_table() -> np.ndarray:
    """Values of all 256 E4M3 codes from torch's float8_e4m3fn decoder."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def exhaustive_check(encoder_address: int, values: np.ndarray, twos: bool, nan_lo: int):
    """Run tests/helpers/code_exhaustive.c over all 2^31 non-negative binary32
    patterns (and their negatives).  Returns (mismatches, first bad pattern)."""
    lib = ctypes.CDLL(build_helper("code_exhaustive"))
    lib.code_check_range.restype = ctypes.c_int64
    lib.code_check_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.POINTER(ctypes.c_uint32)]
    vals = np.ascontiguousarray(values, dtype=np.float64)
    first = ctypes.c_uint32(0)
    bad = lib.code_check_range(0, 1 << 31, encoder_address, vals.ctypes.data_as(ctypes.c_void_p),
                               vals.size, int(twos), nan_lo, cpu_threads(), ctypes.byref(first))
    return int(bad), int(first.value)


def torch_e5m2_table() -> np.ndarray:
    """Values of all 256 E5M2 codes from torch's float8_e5m2 decoder."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e5m2).to(torch.float64).numpy()
