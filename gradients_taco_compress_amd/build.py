"""Build libtaco.so in-tree with hipcc for gfx950.

    python gradients_taco_compress_amd/build.py
    TACO_HIPCC_FLAGS="-DTACO_WAVES_PER_GROUP=8" python gradients_taco_compress_amd/build.py
    TACO_HIPCC_FLAGS="-DTACO_WAVES_PER_GROUP=8" python gradients_taco_compress_amd/build.py \
        --out /tmp/libtaco_wpg8.so

(TACO_HIPCC_FLAGS: extra hipcc flags, e.g. the kernels' compile-time tuning
knobs, for timing a variant with bench.py; unset for the default build.
--out PATH builds only the operator library, to PATH, leaving the in-tree
libraries alone: a variant to time beside the default one with
``python -m gradients_taco_compress_amd.abtime``)

(run as a script: importing it through the package would load the package,
which needs the library this builds)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
#: Translation units: one kernel set per code format, plus the C ABI.
SOURCES = [os.path.join(CSRC, f) for f in
           ("taco_abi.hip", "taco_e4m3.hip", "taco_e5m2.hip", "taco_int8.hip")]
#: Every file the library is built from (sources and headers).
ALL_FILES = SOURCES + [os.path.join(CSRC, "taco_kernels.hpp"),
                       os.path.join(CSRC, "taco_internal.hpp")]
HEADER = os.path.join(ROOT, "include", "taco.h")
LIB = os.path.join(PKG, "libtaco.so")
#: The measurement kernels (not part of the operator), a library of their own.
PROBE_SOURCE = os.path.join(CSRC, "taco_probe.hip")
PROBE_LIB = os.path.join(PKG, "libtaco_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # No packed-FP32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Kernel arguments preloaded into SGPRs (gfx950): a wave starts without
    # loading them from the argument segment.  Same-box A/B, outputs
    # bit-identical: 4 MiB compress / decompress -8 % / -12 %, 40 MiB
    # -2.4 % / -3.5 %, 112 MiB about -1 %.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]

# hipcc's host pass does not know the packed-fp32 feature and says so.
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))


def extra_flags() -> list:
    """Extra hipcc flags from TACO_HIPCC_FLAGS (whitespace-separated)."""
    return os.environ.get("TACO_HIPCC_FLAGS", "").split()


def build(verbose: bool = False, out: str | None = None) -> str:
    """Compile every source (in parallel), link LIB and PROBE_LIB; always
    recompiles.  Returns LIB.  With out, only the operator library is
    built, to that path."""
    from concurrent.futures import ThreadPoolExecutor
    tag = f".tmp{os.getpid()}"
    flags = FLAGS + extra_flags()
    sources = SOURCES + ([] if out else [PROBE_SOURCE])
    lib = os.path.abspath(out) if out else LIB
    objs = [os.path.join(CSRC, os.path.basename(src) + tag + ".o") for src in sources]
    temps = objs + [lib + tag, PROBE_LIB + tag]
    try:
        with ThreadPoolExecutor(max_workers=len(sources)) as pool:
            jobs = [pool.submit(_run, [HIPCC, *flags, "-I", os.path.join(ROOT, "include"),
                                       "-c", src, "-o", obj], verbose)
                    for src, obj in zip(sources, objs)]
            for j in jobs:
                j.result()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", *objs[:len(SOURCES)], "-o", lib + tag],
             verbose)
        if not out:
            _run([HIPCC, "--offload-arch=gfx950", "-shared", objs[-1], "-o", PROBE_LIB + tag],
                 verbose)
        os.replace(lib + tag, lib)
        if not out:
            os.replace(PROBE_LIB + tag, PROBE_LIB)
    finally:
        for path in temps:
            if os.path.exists(path):
                os.remove(path)
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="Build libtaco (and libtaco_probe) for gfx950.")
    ap.add_argument("-q", action="store_true", help="quiet")
    ap.add_argument("--out", default=None,
                    help="build only the operator library, to this path")
    a = ap.parse_args()
    print(build(verbose=not a.q, out=a.out))
