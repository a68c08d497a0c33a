"""Same-box A/B timing of libtaco builds: builds that differ only in a
compile-time tuning knob (or a source change) are loaded side by side and
their kernels timed interleaved in one process, so that the comparison does
not carry the 1-3 % that separate two runs or two boxes.

    TACO_HIPCC_FLAGS="-DTACO_WAVES_PER_GROUP=8" \\
        python gradients_taco_compress_amd/build.py --out /tmp/libtaco_wpg8.so
    python -m gradients_taco_compress_amd.abtime --workload gpt2.7b_rowpar_8192x2560 \\
        gradients_taco_compress_amd/libtaco.so /tmp/libtaco_wpg8.so

For each build and operation (compress, decompress, decompress_accumulate;
E4M3, separate buffers) a HIP graph of K launches is captured over buffer
sets rotated so that every replay loads at least 1 GiB (four times the
Infinity Cache); after a warmup the graphs are replayed in turn, REPEATS
times each, timed with HIP events on the stream they run on.  Printed: one
JSON line with the median microseconds per launch of each build and
operation, and whether every build gave bit-identical outputs on the
workload (codes, alpha and scale of compress, the bf16 of decompress, the
accumulator of decompress_accumulate).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

OPS = ("compress", "decompress", "accumulate")
ROTATE_LOAD_BYTES = 1 << 30
REPEATS = 15


def load(path: str):
    """A libtaco build by path, with the argument types of the three calls."""
    lib = ctypes.CDLL(os.path.abspath(path))
    P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.taco_compress.argtypes = [P, I64, I64, I32, F32, P, P, P, P]
    lib.taco_decompress.argtypes = [P, P, P, I64, I64, I32, P, P]
    lib.taco_decompress_accumulate.argtypes = [P, P, P, I64, I64, I32, P, P]
    for f in (lib.taco_compress, lib.taco_decompress, lib.taco_decompress_accumulate):
        f.restype = ctypes.c_int
    return lib


def bytes_per_launch(op: str, n: int, block: int) -> int:
    """Algorithmic bytes of one launch on n elements."""
    return n * (9 if op == "accumulate" else 3) + 8 * (n // block)


def launcher(lib, op, bufs, rows, cols, block):
    """One launch of op on one buffer set, on torch's current stream."""
    x, c, a, s, y, acc = bufs

    def run(stream):
        if op == "compress":
            st = lib.taco_compress(x.data_ptr(), rows, cols, block, 1.0, c.data_ptr(),
                                   a.data_ptr(), s.data_ptr(), stream)
        elif op == "decompress":
            st = lib.taco_decompress(c.data_ptr(), a.data_ptr(), s.data_ptr(), rows, cols, block,
                                     y.data_ptr(), stream)
        else:
            st = lib.taco_decompress_accumulate(c.data_ptr(), a.data_ptr(), s.data_ptr(), rows,
                                                cols, block, acc.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"{op} returned status {st}")
    return run


def outputs(torch, lib, bufs, rows, cols, block):
    """(codes, alpha, scale, bf16 output, accumulator) of one build on the
    first buffer set, the accumulator starting from zero."""
    x, c, a, s, y, acc = bufs
    stream = torch.cuda.current_stream().cuda_stream
    acc.zero_()
    for op in OPS:
        launcher(lib, op, bufs, rows, cols, block)(stream)
    torch.cuda.synchronize()
    return [t.clone() for t in (c, a, s, y, acc)]


def compare(libs, workload: str, block: int, ops=OPS, repeats: int = REPEATS,
            rotate_bytes: int = ROTATE_LOAD_BYTES, launches: int | None = None) -> dict:
    """Times ops of every build in libs on a workload (see the module
    docstring); rotate_bytes and launches (per graph) shrink the run for a
    quick check."""
    import numpy as np
    import torch
    import synth
    r = synth.WORKLOADS[workload]
    n, m = r.numel, r.numel // block
    rows, cols = r.rows, r.cols
    x0 = torch.from_numpy(synth.generate(r).view(np.int16)).cuda().view(torch.bfloat16)
    nsets = max(1, -(-rotate_bytes // n))                # the codes: n bytes per set
    sets = []
    for _ in range(nsets):
        sets.append((x0.clone(), torch.empty(n, dtype=torch.uint8, device="cuda"),
                     torch.empty(m, dtype=torch.float32, device="cuda"),
                     torch.empty(m, dtype=torch.float32, device="cuda"),
                     torch.empty(n, dtype=torch.bfloat16, device="cuda"),
                     torch.zeros(n, dtype=torch.float32, device="cuda")))
    loaded = [load(p) for p in libs]
    ref = outputs(torch, loaded[0], sets[0], rows, cols, block)
    identical = all(all(torch.equal(u, v) for u, v in zip(ref, outputs(torch, lib, sets[0], rows,
                                                                       cols, block)))
                    for lib in loaded[1:])
    # Every set holds valid codes before the decompress graphs run.
    stream = torch.cuda.current_stream()
    for bufs in sets:
        launcher(loaded[0], "compress", bufs, rows, cols, block)(stream.cuda_stream)
    torch.cuda.synchronize()
    K = launches or max(nsets, 50, int(2e9 // (3 * n)))
    graphs = {}
    for li, lib in enumerate(loaded):
        for op in ops:
            runs = [launcher(lib, op, sets[i % nsets], rows, cols, block) for i in range(K)]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                h = torch.cuda.current_stream().cuda_stream
                for run in runs:
                    run(h)
            graphs[(li, op)] = g
    for g in graphs.values():
        g.replay()
        g.replay()
    times = {k: [] for k in graphs}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(repeats):
        for k, g in graphs.items():
            g.replay()                                  # back to back with the timed replay
            ev[0].record(stream)
            g.replay()
            ev[1].record(stream)
            ev[1].synchronize()
            times[k].append(ev[0].elapsed_time(ev[1]) * 1e3 / K)
    us = {}
    for (li, op), v in times.items():
        t = statistics.median(v)
        us.setdefault(os.path.basename(libs[li]) if libs.count(libs[li]) == 1 else
                      f"{li}:{os.path.basename(libs[li])}", {})[op] = {
            "us": round(t, 3), "GBps": round(bytes_per_launch(op, n, block) / (t * 1e-6) / 1e9, 1)}
    return {"workload": workload, "block": block, "launches_per_graph": K, "sets": nsets,
            "repeats": repeats, "identical_outputs": identical, "builds": us}


def main(argv=None):
    import synth
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("libs", nargs="+", help="libtaco builds (.so paths)")
    ap.add_argument("--workload", default="gpt2.7b_rowpar_8192x2560", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--block", type=int, default=None, help="block size (default: the workload's first)")
    ap.add_argument("--ops", default=",".join(OPS), help="comma-separated subset of " + ",".join(OPS))
    ap.add_argument("--repeats", type=int, default=REPEATS)
    args = ap.parse_args(argv)
    ops = tuple(o for o in args.ops.split(",") if o)
    if not ops or any(o not in OPS for o in ops):
        ap.error(f"--ops must be a subset of {','.join(OPS)}")
    if args.repeats < 1:
        ap.error("--repeats must be at least 1")
    block = args.block or synth.WORKLOADS[args.workload].blocks[0]
    print(json.dumps(compare(args.libs, args.workload, block, ops, args.repeats)), flush=True)


if __name__ == "__main__":
    main()
