"""Seeded synthetic bf16 inputs for the TACO operator.

Shared by the GPU tests, the oracle tests and the benchmark; it holds none of
the compression arithmetic (see ``synth.c`` for the generator and its recipe).

The five workloads stand in for the TP intermediate tensors of the TACO paper
(section 3.1, Figure 4: zero-centred, concentrated near zero, long-tailed,
with outlier channels); the paper trains on datasets and weights that are not
available here, so these seeded draws take their place.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libtaco_synth.so")
_lib = None

LAPLACE, NORMAL, MIXTURE = 0, 1, 2


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i64, f64 = ctypes.c_int64, ctypes.c_double
        lib.taco_synth_generate.argtypes = [
            ctypes.c_uint64, i64, i64, ctypes.c_int, f64, f64, f64, f64, f64,
            i64, f64, f64, ctypes.c_void_p, ctypes.c_int]
        lib.taco_synth_pick_columns.argtypes = [ctypes.c_uint64, i64, i64, ctypes.c_void_p]
        _lib = lib
    return _lib


@dataclass(frozen=True)
class Recipe:
    """One synthetic tensor: shape, seed and value distribution."""
    name: str
    rows: int
    cols: int
    seed: int
    body: int                 # LAPLACE (p1 = scale b), NORMAL (p1 = std),
    p1: float                 # MIXTURE (p1 = weight of the first component,
    p2: float = 0.0           #          p2 / p3 = the two standard deviations)
    p3: float = 0.0
    p_out: float = 0.0        # fraction of entries replaced by out_scale * t3
    out_scale: float = 1.0
    n_chan: int = 0           # outlier hidden channels (whole columns) ...
    chan_factor: float = 1.0  # ... multiplied by this factor
    p_zero: float = 0.0       # fraction of exact zeros
    blocks: tuple = field(default=(128,))

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    def with_shape(self, rows: int, cols: int | None = None, seed: int | None = None) -> "Recipe":
        """Same distribution at another shape (for scaled-down parity cases)."""
        d = dict(self.__dict__)
        d["rows"] = rows
        if cols is not None:
            d["cols"] = cols
        if seed is not None:
            d["seed"] = seed
        return Recipe(**d)


#: The five workloads.  Distribution parameters: Laplace(0, b) takes the scale
#: b, N(0, s) the standard deviation s.
WORKLOADS = {
    # X[2048,1024]: Laplace(0, 0.02), 0.1% of entries replaced by 0.5 * t3.
    "laplace_2048x1024": Recipe("laplace_2048x1024", 2048, 1024, 0, LAPLACE, 0.02,
                                p_out=1e-3, out_scale=0.5, blocks=(128,)),
    # GPT-2.7B-like row-parallel output X[8192,2560] (micro-batch 4 x seq 2048):
    # Laplace(0, 0.01) body, 4 outlier hidden channels scaled 30x.
    "gpt2.7b_rowpar_8192x2560": Recipe("gpt2.7b_rowpar_8192x2560", 8192, 2560, 1, LAPLACE, 0.01,
                                       n_chan=4, chan_factor=30.0, blocks=(128,)),
    # Qwen-7B-like activation X[16384,3584]: 95% N(0, 0.005) + 5% N(0, 0.1).
    "qwen7b_act_16384x3584": Recipe("qwen7b_act_16384x3584", 16384, 3584, 2, MIXTURE, 0.95,
                                    0.005, 0.1, blocks=(128, 256)),
    # Backward gradient G[8192,8192]: N(0, 1e-4), 8 outlier channels at 50x,
    # 1% exact zeros.
    "grad_8192x8192": Recipe("grad_8192x8192", 8192, 8192, 3, NORMAL, 1e-4,
                             n_chan=8, chan_factor=50.0, p_zero=0.01, blocks=(256,)),
    # GPT-175B hidden size X[32768,12288]: Laplace(0, 0.02) + 0.1% t3 outliers;
    # four independently seeded payloads (seeds 4..7) are accumulated.
    "gpt175b_hidden_32768x12288": Recipe("gpt175b_hidden_32768x12288", 32768, 12288, 4, LAPLACE,
                                         0.02, p_out=1e-3, out_scale=1.0, blocks=(256,)),
}

#: Payload seeds of the accumulate workload.
ACCUMULATE_SEEDS = (4, 5, 6, 7)

#: The workload the benchmark times by default: the largest, four payloads
#: compressed and accumulated.
DEFAULT_WORKLOAD = "gpt175b_hidden_32768x12288"


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def generate(recipe: Recipe, seed: int | None = None, threads: int | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of shape [rows, cols]."""
    lib = _load()
    out = np.empty((recipe.rows, recipe.cols), dtype=np.uint16)
    s = recipe.seed if seed is None else seed
    rc = lib.taco_synth_generate(
        s, recipe.rows, recipe.cols, recipe.body, recipe.p1, recipe.p2, recipe.p3,
        recipe.p_out, recipe.out_scale, recipe.n_chan, recipe.chan_factor, recipe.p_zero,
        out.ctypes.data_as(ctypes.c_void_p), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"synthetic generator failed ({rc})")
    return out


def outlier_columns(recipe: Recipe, seed: int | None = None) -> np.ndarray:
    """The columns the generator scales by ``chan_factor``."""
    lib = _load()
    picked = np.empty(max(recipe.n_chan, 1), dtype=np.int64)
    s = recipe.seed if seed is None else seed
    if recipe.n_chan and lib.taco_synth_pick_columns(s, recipe.cols, recipe.n_chan,
                                                     picked.ctypes.data_as(ctypes.c_void_p)):
        raise RuntimeError("column pick failed")
    return np.sort(picked[:recipe.n_chan])


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 view of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bits(values) -> np.ndarray:
    """bf16 bit patterns of float32 values (nearest-even; values are expected to be finite)."""
    u = np.asarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)
