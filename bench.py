#!/usr/bin/env python3
"""Benchmark of the TACO compression operator on one MI355X.

One step = one pass of the whole operator over one batch of synthetic input:
four ``taco_compress`` + four ``taco_decompress_accumulate`` calls for the
four-payload workload X[32768,12288] (the default line, the largest
workload), or ``taco_compress`` then ``taco_decompress`` (the round trip) for
the round-trip workloads, which the default line reports under ``configs``
(each timed after its own warmup, never part of ``value``).
Inputs are resident in HBM before timing starts.  Buffer sets are rotated so
that every timed graph loads more than 1 GiB per replay (four times the
256 MB Infinity Cache) and each kernel streams its inputs from HBM.  The timed steps are replayed from a
HIP graph so that host launch overhead does not gap the GPU.

Prints one JSON line (rank 0, the only rank): the headline metric is input
GB/s of bf16 (2 bytes per element) per round trip, plus a roofline object for
the dominant kernel and the CPU oracle's rate on the same workload.

    python bench.py [--steps K] [--warmup W]      # exactly W warmup and K timed steps
    python bench.py --workload NAME[:variant] [--block B]
    python bench.py --all --out results.json     # every workload (stderr table)

``NAME:owner`` times the fused owner step of the two-shot all-reduce
(``taco_reduce_compress`` of an own partial plus three payloads) instead,
``NAME:owner_packed`` the same on interleaved records;
``NAME:packed`` the round trip through the interleaved wire layout;
``NAME:e5m2`` and ``NAME:int8`` the round trip with E5M2 or INT8 codes;
``NAME:accn`` (the four-payload workload) sums the four payloads with one
``taco_decompress_accumulate_n`` call instead of four accumulates;
``NAME:fidelity`` the fidelity study's fused round trip (``taco_roundtrip``,
the operator's variant, error sums only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compress+decompress GB/s of bf16 input and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak (AMD specification), GB/s
MALL_BYTES = 256 << 20
# Buffer sets rotate so that every timed graph LOADS at least this much per
# replay (four times the 256 MB Infinity Cache): data that cached loads leave
# in the cache is long evicted when it is read again, so every kernel
# streams its inputs from HBM.
ROTATE_LOAD_BYTES = 4 * MALL_BYTES
MAX_SET_BYTES = 12 << 30


def rotation_sets(min_load_bytes: int, set_bytes: int) -> int:
    """Buffer sets so that the smallest per-set load, repeated, reaches
    ROTATE_LOAD_BYTES (capped by device memory)."""
    nsets = max(1, -(-ROTATE_LOAD_BYTES // max(1, min_load_bytes)))
    return max(1, min(nsets, MAX_SET_BYTES // max(1, set_bytes)))
KERNEL_DIR = os.path.join(ROOT, "gradients_taco_compress_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
VALU_FILE = os.path.join(ROOT, "profiles", "valu_insts.json")
# VALU issue peak of MI355X: a wave64 VALU instruction occupies a 16-lane SIMD
# for 4 cycles; 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-instructions/s
# (non-packed 32-bit VALU).
VALU_PEAK_LANE_INSTR = 256 * 4 * 16 * 2.4e9


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default: 100 for the four-payload workload, 400 for the "
                        "round trips)")
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps right before the timed ones (default: one pass over "
                        "every buffer set, at least 20)")
    p.add_argument("--workload", default=None)
    p.add_argument("--block", type=int, default=None)
    p.add_argument("--all", action="store_true", help="time every workload and block size")
    p.add_argument("--out", default=None, help="also write the JSON record(s) to this file")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-floors", action="store_true",
                   help="skip the launch / stream floors and the same-mix reference (for "
                        "counter runs, where every dispatch is slow)")
    p.add_argument("--no-configs", action="store_true",
                   help="default line only: skip the round trips of the other workloads "
                        "(reported under 'configs')")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU seconds of each leg of the oracle baseline")
    p.add_argument("--torch-reference", action="store_true",
                   help="time torch's elementwise add and copy over the same bytes as each "
                        "workload's compress (context for the roofline) and exit")
    p.add_argument("--copy-probe", action="store_true",
                   help="run only a plain device copy of known size (HBM counter calibration)")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    return p.parse_args()


def algorithmic_bytes(op: str, n: int, block: int) -> float:
    """Bytes the operator must move: bf16 in/out 2/elem, codes 1/elem,
    alpha + s 8 bytes per block, float32 accumulator 4 + 4 per element."""
    side = 8.0 * n / block
    if op.startswith("reduce_compress"):
        npay = int(op.split(":")[1]) if ":" in op else 3
        return 2.0 * n + npay * (n + side) + n + side
    if op == "compress":
        return 2.0 * n + n + side
    if op == "decompress":
        return n + side + 2.0 * n
    if op == "accumulate":
        return n + side + 8.0 * n
    if op == "roundtrip":
        return 2.0 * n
    if op.startswith("accumulate_n"):
        npay = int(op.split(":")[1])
        return npay * (n + side) + 8.0 * n
    raise ValueError(op)


#: libtaco's sources (the measurement kernels of libtaco_probe are not part of it).
LIBTACO_SOURCES = ("taco_abi.hip", "taco_e4m3.hip", "taco_e5m2.hip", "taco_int8.hip",
                   "taco_internal.hpp", "taco_kernels.hpp")


def build_flags() -> list:
    """The hipcc flags of the default build (build.py's FLAGS), read without
    importing the package."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_taco_build_flags", os.path.join(os.path.dirname(KERNEL_DIR), "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return list(mod.FLAGS)


def kernel_hash() -> str:
    """sha256[:16] over libtaco's sources (file names and contents, sorted)
    and the compile flags of the default build: the committed counter runs
    count only while the code they were taken on is the code that runs."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_DIR)):
        if name in LIBTACO_SOURCES:
            h.update(name.encode())
            with open(os.path.join(KERNEL_DIR, name), "rb") as f:
                h.update(f.read())
    h.update(("flags:" + " ".join(build_flags())).encode())
    return h.hexdigest()[:16]


def valu_for(kernel: str, workload: str, block: int):
    """VALU wave-instructions per launch from the committed rocprofv3 counter
    run (SQ_INSTS_VALU), if taken on the current kernel source; else None."""
    try:
        with open(VALU_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    e = t.get("entries", {}).get(f"{kernel}:{workload}:{block}")
    return None if e is None else e.get("sq_insts_valu")


def valu_roofline(insts: float, seconds: float) -> dict:
    """VALU issue rate of a launch against the issue peak."""
    achieved = insts * 64 / seconds
    return {"bound": "alu", "achieved": round(achieved / 1e12, 2),
            "peak": round(VALU_PEAK_LANE_INSTR / 1e12, 2), "unit": "T lane-instr/s",
            "frac": round(achieved / VALU_PEAK_LANE_INSTR, 4),
            "wave_instructions": insts}


def traffic_for(kernel: str, workload: str, block: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    e = t.get("entries", {}).get(f"{kernel}:{workload}:{block}")
    return None if e is None else e.get("hbm_bytes_per_launch")


class Timer:
    """HIP events on the stream the kernels run on."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def time(self, fn, reps: int) -> float:
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(self.stream)
        for _ in range(reps):
            fn()
        b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b) * 1e-3          # seconds


def make_graph(torch, fn, use_graph: bool, prerun: bool = True):
    """fn captured into a HIP graph (returns its replay).  prerun runs fn once
    eagerly before the capture (lazy initialisation of torch's own kernels);
    libtaco's launches need none, and the operator's step graphs skip it so
    that no step runs outside the counted warmup and timed steps."""
    if not use_graph:
        return fn
    if prerun:
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g.replay


STEP_CHUNK = 2048      # most steps captured into one HIP graph


def run_cycle(torch, sets, one, count: int, use_graph: bool):
    """A callable that runs one(set) for exactly `count` consecutive steps,
    cycling through the buffer sets, as HIP graphs of at most STEP_CHUNK
    steps (a full graph replayed, then a remainder graph)."""
    if count <= 0:
        return lambda: None

    def body(c):
        def run():
            for i in range(c):
                one(sets[i % len(sets)])
        return run

    chunk = min(count, STEP_CHUNK)
    q, rem = divmod(count, chunk)
    full = make_graph(torch, body(chunk), use_graph, prerun=False)
    tail = make_graph(torch, body(rem), use_graph, prerun=False) if rem else None

    def go():
        for _ in range(q):
            full()
        if tail is not None:
            tail()
    return go


# The GPU's clocks ramp up during its first milliseconds of work after idle
# time: measured on the 40 MiB round trip, a 10 ms graph replay that follows
# 5-500 ms of host-side idling runs 5-9 % slower than back-to-back replays,
# and about 10 ms of continuous work restores the steady rate.  So the default
# warmup is continuous (replayed from graphs, like the timed steps) and moves
# at least this many algorithmic bytes (about 20 ms at 5 TB/s).
WARM_BYTES = 100e9
# Replays of the K timed steps after the timed region, for the spread.
REPEATS = 20


def warmup_steps(warmup, nsets: int, step_bytes: float) -> int:
    """Untimed steps: as asked; by default enough to move WARM_BYTES, at least
    one pass over every buffer set and at least 20."""
    if warmup is not None:
        return warmup
    return max(20, nsets, int(-(-WARM_BYTES // step_bytes)))


def time_steps(torch, sets, step_one, kernels: dict, steps: int, warmup, use_graph: bool,
               step_bytes: float):
    """The graphs are captured first (capture runs nothing on the GPU); then
    exactly `warmup` untimed steps replay back to back, right before exactly
    `steps` timed steps (seconds per step).  Then each kernel alone over at
    least one pass of the sets and at least WARM_BYTES / 4 of its step's bytes
    (seconds per launch, after one untimed pass of the same graph), for its
    roofline.  After the timed steps, REPEATS more replays of the same K
    steps give the spread of the measurement (reported beside the value,
    never in it).  Returns (t_step, per_kernel, warmup steps run, seconds
    per step of each repeat)."""
    timer = Timer(torch)
    warm = warmup_steps(warmup, len(sets), step_bytes)
    warm_fn = run_cycle(torch, sets, step_one, warm, use_graph)
    step_fn = run_cycle(torch, sets, step_one, steps, use_graph)
    count = max(steps, len(sets), int(-(-WARM_BYTES // (4 * step_bytes))))
    kernel_fns = {k: run_cycle(torch, sets, one, count, use_graph) for k, one in kernels.items()}
    warm_fn()
    t_step = timer.time(step_fn, 1) / steps
    repeats = [timer.time(step_fn, 1) / steps for _ in range(REPEATS)]
    per_kernel = {}
    for kname, fn in kernel_fns.items():
        fn()
        per_kernel[kname] = timer.time(fn, 1) / count
    return t_step, per_kernel, warm, repeats


def roundtrip_case(torch, taco, synth, name: str, block: int, steps: int, warmup,
                   use_graph: bool, fmt: str = "e4m3"):
    import numpy as np
    r = synth.WORKLOADS[name]
    n = r.numel
    x_bits = synth.generate(r)
    x0 = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    m = n // block
    per_set = 2 * n + n + 8 * m + 2 * n
    nsets = rotation_sets(n + 8 * m, per_set)        # the codes are the smallest input
    sets = []
    for _ in range(nsets):
        x = x0.clone()
        codes = torch.empty((r.rows, r.cols), dtype=torch.uint8, device="cuda")
        alpha = torch.empty(m, dtype=torch.float32, device="cuda")
        scale = torch.empty(m, dtype=torch.float32, device="cuda")
        y = torch.empty((r.rows, r.cols), dtype=torch.bfloat16, device="cuda")
        sets.append((x, codes, alpha, scale, y))
    del x0

    def one_compress(st):
        x, codes, alpha, scale, _ = st
        taco.compress(x, block=block, codes=codes, alpha=alpha, scale=scale, fmt=fmt)

    def one_decompress(st):
        _, codes, alpha, scale, y = st
        taco.decompress(codes, alpha, scale, block=block, out=y, fmt=fmt)

    def one_step(st):
        one_compress(st)
        one_decompress(st)

    step_bytes = algorithmic_bytes("compress", n, block) + algorithmic_bytes("decompress", n, block)
    t_step, kt, warm, reps = time_steps(torch, sets, one_step,
                                  {"compress": one_compress, "decompress": one_decompress},
                                  steps, warmup, use_graph, step_bytes)
    t_c, t_d = kt["compress"], kt["decompress"]
    return {"n": n, "block": block, "steps": steps, "warmup": warm, "t_step": t_step,
            "repeats": reps, "t_compress": t_c, "t_decompress": t_d, "sets": nsets, "rows": r.rows, "cols": r.cols, "format": fmt,
            "bytes_step": algorithmic_bytes("compress", n, block)
            + algorithmic_bytes("decompress", n, block),
            "input_bytes_step": 2.0 * n, "kernels": {"compress": t_c, "decompress": t_d}}


def packed_case(torch, taco, synth, name: str, block: int, steps: int, warmup,
                use_graph: bool):
    """Round trip through the interleaved wire layout (one payload buffer per
    direction, codes and scalars together)."""
    import numpy as np
    r = synth.WORKLOADS[name]
    n = r.numel
    m = n // block
    x0 = torch.from_numpy(synth.generate(r).view(np.int16)).cuda().view(torch.bfloat16)
    nbytes = taco.taco_packed_bytes(r.rows, r.cols, block)
    per_set = 2 * n + nbytes + 2 * n
    nsets = rotation_sets(nbytes, per_set)
    sets = [(x0.clone(), torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
             torch.empty((r.rows, r.cols), dtype=torch.bfloat16, device="cuda")) for _ in range(nsets)]
    del x0

    def one_compress(st):
        x, pay, _ = st
        taco.compress_packed(x, block=block, payload=pay)

    def one_decompress(st):
        _, pay, y = st
        taco.decompress_packed(pay, y.shape, block=block, out=y)

    def one_step(st):
        one_compress(st)
        one_decompress(st)

    step_bytes = (algorithmic_bytes("compress", n, block)
                  + algorithmic_bytes("decompress", n, block))
    t_step, kt, warm, reps = time_steps(torch, sets, one_step,
                                  {"compress": one_compress, "decompress": one_decompress},
                                  steps, warmup, use_graph, step_bytes)
    t_c, t_d = kt["compress"], kt["decompress"]
    return {"n": n, "block": block, "steps": steps, "warmup": warm, "t_step": t_step,
            "repeats": reps, "sets": nsets, "rows": r.rows, "cols": r.cols, "packed": True,
            "bytes_step": algorithmic_bytes("compress", n, block)
            + algorithmic_bytes("decompress", n, block),
            "input_bytes_step": 2.0 * n, "kernels": {"compress": t_c, "decompress": t_d}}


def fidelity_case(torch, taco, synth, name: str, block: int, steps: int, warmup,
                  use_graph: bool):
    """taco_roundtrip of the operator's variant with error sums only: reads
    the bf16 tensor once (plus a clearing launch of the 40-byte sums)."""
    import numpy as np
    r = synth.WORKLOADS[name]
    n = r.numel
    x0 = torch.from_numpy(synth.generate(r).view(np.int16)).cuda().view(torch.bfloat16)
    nsets = rotation_sets(2 * n, 2 * n)
    sets = [(x0.clone(), torch.empty(taco.FIDELITY_SUMS_BYTES, dtype=torch.uint8, device="cuda"))
            for _ in range(nsets)]
    del x0

    def one_step(st):
        x, sums = st
        taco.roundtrip(x, block=block, variant="taco", sums=sums)

    t, _, warm, reps = time_steps(torch, sets, one_step, {}, steps, warmup, use_graph, 2.0 * n)
    return {"n": n, "block": block, "steps": steps, "warmup": warm, "t_step": t, "sets": nsets,
            "repeats": reps, "rows": r.rows, "cols": r.cols, "fidelity": True, "bytes_step": 2.0 * n,
            "input_bytes_step": 2.0 * n,
            "kernels": {"roundtrip": t}}


def accumulate_case(torch, taco, synth, name: str, block: int, steps: int, warmup,
                    use_graph: bool, fused: bool = False, also_fused: bool = False):
    """Four payloads compressed and summed into one float32 accumulator: one
    taco_decompress_accumulate per payload, or (fused) one
    taco_decompress_accumulate_n over all four.  also_fused: after the timed
    steps, time the fused form too on the same resident payloads (reported
    beside the line, never in its value)."""
    import numpy as np
    r = synth.WORKLOADS[name]
    n = r.numel
    m = n // block
    payloads = []
    for seed in synth.ACCUMULATE_SEEDS:
        x_bits = synth.generate(r, seed=seed)
        x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        del x_bits
        codes = torch.empty((r.rows, r.cols), dtype=torch.uint8, device="cuda")
        alpha = torch.empty(m, dtype=torch.float32, device="cuda")
        scale = torch.empty(m, dtype=torch.float32, device="cuda")
        payloads.append((x, codes, alpha, scale))
    acc = torch.zeros((r.rows, r.cols), dtype=torch.float32, device="cuda")

    def run_compress():
        for x, codes, alpha, scale in payloads:
            taco.compress(x, block=block, codes=codes, alpha=alpha, scale=scale)

    def run_accumulate():
        if fused:
            taco.decompress_accumulate_n([(c, a, s) for _, c, a, s in payloads], acc, block=block)
            return
        for _, codes, alpha, scale in payloads:
            taco.decompress_accumulate(codes, alpha, scale, acc, block=block)

    def run_steps():
        run_compress()
        run_accumulate()

    # Graphs first, then exactly `warm` untimed steps, then the timed steps
    # (as in time_steps); each kernel graph gets one untimed replay first.
    nb = len(payloads)
    acc_bytes = (algorithmic_bytes(f"accumulate_n:{nb}", n, block) if fused
                 else nb * algorithmic_bytes("accumulate", n, block))
    step_bytes = nb * algorithmic_bytes("compress", n, block) + acc_bytes
    step_fn = make_graph(torch, run_steps, use_graph, prerun=False)
    comp_fn = make_graph(torch, run_compress, use_graph, prerun=False)
    acc_fn = make_graph(torch, run_accumulate, use_graph, prerun=False)
    warm = warmup_steps(warmup, 1, step_bytes)
    for _ in range(warm):                 # graph replays: back to back on the GPU
        step_fn()
    reps = max(1, steps)
    timer = Timer(torch)
    t_steps = timer.time(step_fn, reps)
    repeats = [timer.time(step_fn, reps) / reps for _ in range(REPEATS)]
    comp_fn()
    t_c = timer.time(comp_fn, reps) / (nb * reps)
    acc_fn()
    t_a = timer.time(acc_fn, reps) / ((1 if fused else nb) * reps)
    kname = "accumulate_n" if fused else "accumulate"
    out = {"n": n, "block": block, "steps": reps, "warmup": warm, "t_step": t_steps / reps,
           "repeats": repeats, "t_compress": t_c, "t_accumulate": t_a, "sets": 1, "rows": r.rows, "cols": r.cols,
           "fused": fused, "nb": nb,
           "bytes_step": nb * algorithmic_bytes("compress", n, block) + acc_bytes,
           "input_bytes_step": nb * 2.0 * n, "kernels": {"compress": t_c, kname: t_a}}
    if also_fused and not fused:
        def run_fused():
            run_compress()
            taco.decompress_accumulate_n([(c, a, s) for _, c, a, s in payloads], acc, block=block)
        fused_fn = make_graph(torch, run_fused, use_graph, prerun=False)
        accn_fn = make_graph(torch, lambda: taco.decompress_accumulate_n(
            [(c, a, s) for _, c, a, s in payloads], acc, block=block), use_graph, prerun=False)
        fbytes = nb * algorithmic_bytes("compress", n, block) + \
            algorithmic_bytes(f"accumulate_n:{nb}", n, block)
        for _ in range(warmup_steps(None, 1, fbytes)):
            fused_fn()
        t_f = timer.time(fused_fn, reps) / reps
        accn_fn()
        t_n = timer.time(accn_fn, reps) / reps
        out["fused_receive"] = {
            "step": f"{nb}x compress + 1x decompress_accumulate_n of {nb} payloads",
            "steps": reps, "ms_per_step": round(t_f * 1e3, 5),
            "input_GBps": round(nb * 2.0 * n / t_f / 1e9, 2),
            "pct_hbm_peak": round(100.0 * fbytes / t_f / 1e9 / HBM_PEAK_GBS, 2),
            "kernel_us": {"compress": round(t_c * 1e6, 3), "accumulate_n": round(t_n * 1e6, 3)}}
    return out


def owner_case(torch, taco, synth, name: str, block: int, steps: int, warmup,
               use_graph: bool, packed: bool = False):
    """Owner step of the two-shot all-reduce: own bf16 partial plus three
    received payloads (four independently seeded tensors) reduced and
    compressed again in one taco_reduce_compress call (with packed, on
    interleaved records: taco_reduce_compress_packed)."""
    import numpy as np
    r = synth.WORKLOADS[name]
    n = r.numel
    m = n // block
    seeds = synth.ACCUMULATE_SEEDS
    own = torch.from_numpy(synth.generate(r, seed=seeds[0]).view(np.int16)).cuda().view(torch.bfloat16)
    pay = []
    for seed in seeds[1:]:
        x = torch.from_numpy(synth.generate(r, seed=seed).view(np.int16)).cuda().view(torch.bfloat16)
        pay.append(taco.compress_packed(x, block=block) if packed else taco.compress(x, block=block))
        del x
    codes = torch.empty((r.rows, r.cols), dtype=torch.uint8, device="cuda")
    alpha = torch.empty(m, dtype=torch.float32, device="cuda")
    scale = torch.empty(m, dtype=torch.float32, device="cuda")
    out = torch.empty(taco.taco_packed_bytes(r.rows, r.cols, block), dtype=torch.uint8,
                      device="cuda") if packed else None

    def run_steps():
        if packed:
            taco.reduce_compress_packed(own, pay, block=block, out=out)
        else:
            taco.reduce_compress(own, pay, block=block, codes=codes, alpha=alpha, scale=scale)

    npay = len(pay)
    kbytes = 2.0 * n + npay * (n + 8.0 * n / block) + n + 8.0 * n / block
    step_fn = make_graph(torch, run_steps, use_graph, prerun=False)
    warm = warmup_steps(warmup, 1, kbytes)
    for _ in range(warm):                 # graph replays: back to back on the GPU
        step_fn()
    reps = max(1, steps)
    timer = Timer(torch)
    t = timer.time(step_fn, reps) / reps
    repeats = [timer.time(step_fn, reps) / reps for _ in range(REPEATS)]
    return {"n": n, "block": block, "steps": reps, "warmup": warm, "t_step": t, "sets": 1,
            "repeats": repeats, "rows": r.rows, "cols": r.cols, "bytes_step": kbytes, "input_bytes_step": 2.0 * n,
            "kernels": {"reduce_compress": t}, "npayloads": npay, "packed": packed}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _oracle_rate(oracle, parts, block: int, accumulate: bool, min_seconds: float, pool):
    """Round trips of the oracle over the row parts (concurrently when a
    thread pool is given: each part is one C call, which releases the GIL),
    repeated until min_seconds have passed.  Returns (reps, seconds)."""
    import numpy as np

    def one(part):
        codes, alpha, scale = oracle.compress(part, block)
        if accumulate:
            oracle.decompress_accumulate(codes, alpha, scale, block,
                                         np.zeros(part.size, np.float32))
        else:
            oracle.decompress(codes, alpha, scale, block)

    reps, t = 0, 0.0
    t0 = time.perf_counter()
    while t < min_seconds or reps == 0:
        if pool is None:
            for part in parts:
                one(part)
        else:
            list(pool.map(one, parts))
        reps += 1
        t = time.perf_counter() - t0
    return reps, t


def cpu_baseline(synth, name: str, block: int, min_seconds: float, accumulate: bool):
    """The oracle (plain C, double precision, unchanged) on a bounded sample
    of the same workload: once on one thread, then with the sample's rows
    split over the host's cores (at most 16, the CPU share of one GPU), one
    oracle call per part and thread.  About min_seconds of CPU time each."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    r = synth.WORKLOADS[name]
    rows = r.rows
    if r.numel > (1 << 26):                       # bounded sample: whole rows, <= 64 Mi elements
        rows = max(1, (1 << 26) // r.cols)
    sample = r.with_shape(rows)
    x = synth.generate(sample)
    n = x.size
    oracle.compress(x[:1], block)                 # build / load the library once
    reps1, t1 = _oracle_rate(oracle, [x], block, accumulate, min_seconds, None)
    threads = max(1, min(16, len(os.sched_getaffinity(0)), rows))
    parts = np.array_split(x, threads, axis=0)
    with ThreadPoolExecutor(threads) as pool:
        repsn, tn = _oracle_rate(oracle, parts, block, accumulate,
                                 max(1.0, min_seconds / threads), pool)
    op = "accumulate" if accumulate else "decompress"
    host = os.cpu_count() or 0
    return {"value": 2.0 * n * repsn / tn / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "host_cores": host, "available_cores": len(os.sched_getaffinity(0)),
            "single_thread_value": 2.0 * n * reps1 / t1 / 1e9,
            "sample": f"{rows}x{r.cols} rows of {name} (seed {r.seed}), block {block}; "
                      f"{repsn} x (compress + {op}) in {tn:.1f} s on {threads} threads "
                      f"(rows split evenly; at most 16, the CPU share of one GPU, of the "
                      f"host's {host} cores), {reps1} x in {t1:.1f} s on one thread; "
                      f"{_cpu_model()}"}


def repeat_stats(res):
    """Spread of the measurement: the K timed steps replayed REPEATS more
    times after the timed region (not part of `value`)."""
    r = sorted(res.get("repeats") or [])
    if not r:
        return None
    mid = len(r) // 2
    med = r[mid] if len(r) % 2 else 0.5 * (r[mid - 1] + r[mid])

    def pct(t):
        return round(100.0 * res["bytes_step"] / t / 1e9 / HBM_PEAK_GBS, 2)
    return {"n": len(r), "ms_per_step_median": round(med * 1e3, 5),
            "ms_per_step_min": round(r[0] * 1e3, 5), "ms_per_step_max": round(r[-1] * 1e3, 5),
            "pct_hbm_peak_median": pct(med)}


def record(res, name: str, args, cpu=None):
    t_step = res["t_step"]
    value = res["input_bytes_step"] / t_step / 1e9
    kern = max(res["kernels"], key=lambda k: res["kernels"][k])
    dur = res["kernels"][kern]
    op = (f"reduce_compress:{res['npayloads']}" if kern == "reduce_compress"
          else f"accumulate_n:{res['nb']}" if kern == "accumulate_n" else kern)
    kbytes = algorithmic_bytes(op, res["n"], res["block"])
    achieved = kbytes / dur / 1e9
    fmt = res.get("format", "e4m3")
    key = kern if fmt == "e4m3" else f"{kern}[{fmt}]"
    if res.get("packed"):
        key += "[packed]"           # counters are taken for the side-buffer kernels only
    traffic = traffic_for(key, name, res["block"])
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": res["warmup"],
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "tokens": res["rows"], "hidden": res["cols"],
                   "block": res["block"], "target_energy": 1.0, "format": fmt,
                   "step": ("4x compress + 1x decompress_accumulate_n of 4 payloads"
                            if res.get("fused")
                            else "4x compress + 4x decompress_accumulate" if "t_accumulate" in res
                            else (f"reduce_compress{'_packed' if res.get('packed') else ''} "
                                  f"of own + {res['npayloads']} payloads")
                            if "npayloads" in res
                            else "compress_packed + decompress_packed" if res.get("packed")
                            else "roundtrip with error sums (fidelity study)"
                            if res.get("fidelity")
                            else "compress + decompress"),
                   "buffer_sets": res["sets"], "graph": not args.no_graph},
        "pct_hbm_peak": round(100.0 * res["bytes_step"] / t_step / 1e9 / HBM_PEAK_GBS, 2),
        "repeats": repeat_stats(res),
        "kernel_us": {k: round(v * 1e6, 3) for k, v in res["kernels"].items()},
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": kbytes,
                     "traffic": traffic},
    }
    valu = valu_for(key, name, res["block"]) if fmt == "e4m3" and not res.get("packed") else None
    if valu is not None:
        rec["roofline"]["valu"] = valu_roofline(valu, dur)
    if res.get("fidelity"):
        # The study's round trip keeps the codes in registers and reads the
        # tensor once: it is bound by VALU issue, not by HBM.
        hbm = rec["roofline"]
        rec["roofline"] = dict(valu_roofline(valu, dur) if valu is not None else
                               {"bound": "alu", "achieved": None,
                                "peak": round(VALU_PEAK_LANE_INSTR / 1e12, 2),
                                "unit": "T lane-instr/s", "frac": None},
                               kernel=kern, traffic=hbm["traffic"],
                               hbm={"achieved": hbm["achieved"], "peak": hbm["peak"],
                                    "unit": hbm["unit"], "frac": hbm["frac"]})
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    return rec


def copy_probe(torch):
    """A plain device-to-device copy of 1 GiB, for HBM counter calibration."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def add_reference(torch, n: int, use_graph: bool) -> dict:
    """torch's bf16 elementwise add over N/2-element operands: reads 2N bytes
    and writes N, the byte mix of compress, timed like the operator's kernels
    (buffer sets rotated over more than 1 GiB of loads, HIP graphs, events)."""
    timer = Timer(torch)
    nsets = rotation_sets(2 * n, 3 * n)
    sets = [tuple(torch.ones(n // 2, dtype=torch.bfloat16, device="cuda") for _ in range(3))
            for _ in range(nsets)]

    def add_all():
        for a, b, c in sets:
            torch.add(a, b, out=c)
    fn = make_graph(torch, add_all, use_graph)
    for _ in range(int(-(-WARM_BYTES // (3 * n * nsets)))):    # continuous warmup, untimed
        fn()
    t = timer.time(fn, 20) / (20 * nsets)
    del sets, fn
    torch.cuda.empty_cache()
    return {"bytes": 3 * n, "us": round(t * 1e6, 3), "GBps": round(3 * n / t / 1e9, 1)}


def launch_groups(n: int, block: int) -> int:
    """Work-groups of libtaco's compress / decompress launch on n elements
    (four wavefronts each; one wave-step of 64 / LPB blocks per wavefront,
    LPB = 4, 8, 8, 8, 16 lanes per block for B = 32 ... 512; two wave-steps
    per wavefront at B <= 64 from 16384 wave-steps up)."""
    lpb = {32: 4, 64: 8, 128: 8, 256: 8, 512: 16}[block]
    steps = -(-(n // block) // (64 // lpb))
    if block <= 64 and steps >= 16384:
        steps = -(-steps // 2)
    return max(1, -(-steps // 4))


def launch_floor(torch, probe, groups: int, use_graph: bool, count: int = 2000) -> dict:
    """An empty kernel on the same grid, `count` launches back to back (one
    graph, one untimed replay first): what any launch of that shape costs."""
    timer = Timer(torch)
    fn = make_graph(torch, lambda: [probe.empty(groups) for _ in range(count)], use_graph)
    fn()
    t = timer.time(fn, 1) / count
    return {"kernel": "empty", "groups": groups, "us": round(t * 1e6, 3)}


def stream_floor(torch, probe, mix: str, n: int, algorithmic_bytes_: float, kernel_s: float,
                 use_graph: bool, valu: int = 0) -> dict:
    """A plain stream of the kernel's byte mix over the same number of
    elements (16-byte non-temporal loads and stores, 1 KiB per instruction;
    libtaco_probe), timed like the operator's kernels: buffer sets rotated
    over more than 1 GiB of loads, graphs, a continuous warmup.  Its rate is
    the streaming ceiling a single launch of that size reaches.  With valu >
    0 each wavefront also issues that many dependent VALU instructions
    between its loads and its stores."""
    ld, sto = probe.MIXES[mix]
    waves = max(1, n // 1024)
    load_bytes, store_bytes = waves * ld * 1024, waves * sto * 1024
    nsets = rotation_sets(load_bytes, load_bytes + store_bytes)
    sets = [(torch.ones(load_bytes // 2, dtype=torch.bfloat16, device="cuda"),
             torch.empty(store_bytes, dtype=torch.uint8, device="cuda")) for _ in range(nsets)]
    timer = Timer(torch)
    count = max(20, int(-(-WARM_BYTES // (4 * (load_bytes + store_bytes)))))

    def run():
        for i in range(count):
            src, dst = sets[i % nsets]
            probe.stream(mix, src, dst, waves, valu)
    fn = make_graph(torch, run, use_graph, prerun=False)
    for _ in range(3):                      # continuous warmup
        fn()
    t = timer.time(fn, 1) / count
    del sets, fn
    torch.cuda.empty_cache()
    moved = load_bytes + store_bytes
    rate = moved / t / 1e9
    # The kernel's algorithmic bytes add the per-block scalars (8 / B bytes
    # per element) to the same mix: compare rates, not times.
    what = f"plain stream, {ld} KiB in / {sto} KiB out per wavefront ({mix} mix)"
    if valu:
        what += f", {valu} dependent VALU instructions per wavefront"
    return {"kernel": what, "bytes": moved, "us": round(t * 1e6, 3), "GBps": round(rate, 1),
            "frac": round(rate / HBM_PEAK_GBS, 4),
            "kernel_rate_vs_stream": round((algorithmic_bytes_ / kernel_s) / (moved / t), 4)}


def torch_reference(torch, synth, cases, use_graph: bool):
    """Context for the roofline: torch's own elementwise kernels moving the
    same bytes as compress at each workload's size (add of two bf16 halves:
    reads 2N bytes, writes N, the compress mix 2:1) and a plain bf16 copy
    (reads 2N, writes 2N), timed like the operator's kernels (buffer sets
    rotated over more than 1 GiB of loads, HIP graphs, events).  One JSON
    line per workload."""
    timer = Timer(torch)
    for name, _block in cases:
        n = synth.WORKLOADS[name.split(":")[0]].numel
        out = {"torch_reference": name, "elements": n}
        out["add_2to1"] = add_reference(torch, n, use_graph)
        nsets = rotation_sets(2 * n, 4 * n)
        sets = [(torch.ones(n, dtype=torch.bfloat16, device="cuda"),
                 torch.empty(n, dtype=torch.bfloat16, device="cuda")) for _ in range(nsets)]

        def copy_all():
            for a, c in sets:
                c.copy_(a)
        fn = make_graph(torch, copy_all, use_graph)
        t = timer.time(fn, 20) / (20 * nsets)
        out["copy_1to1"] = {"bytes": 4 * n, "us": round(t * 1e6, 3),
                            "GBps": round(4 * n / t / 1e9, 1)}
        del sets, fn
        torch.cuda.empty_cache()
        print(json.dumps(out), flush=True)


#: The round-trip workloads reported under "configs" beside the default line
#: (each block size of each workload).
ROUNDTRIP_CONFIGS = [("laplace_2048x1024", 128), ("gpt2.7b_rowpar_8192x2560", 128),
                     ("qwen7b_act_16384x3584", 128), ("qwen7b_act_16384x3584", 256),
                     ("grad_8192x8192", 256)]
#: Default timed steps: the four-payload step takes about 3 ms, a round trip
#: 7-70 us.
DEFAULT_STEPS_ACCUMULATE = 100
DEFAULT_STEPS_ROUNDTRIP = 400


def run_case(torch, taco, synth, name: str, block: int, steps, warmup, use_graph: bool,
             also_fused: bool = False):
    """Times one workload (NAME or NAME:variant).  Returns (res, base name,
    accumulate workload?)."""
    base = name.split(":")[0]
    kind = name.split(":")[1] if ":" in name else ""
    acc = base == "gpt175b_hidden_32768x12288" and kind in ("", "accn")
    if steps is None:
        steps = DEFAULT_STEPS_ACCUMULATE if acc or kind.startswith("owner") \
            else DEFAULT_STEPS_ROUNDTRIP
    if kind in ("owner", "owner_packed"):
        res = owner_case(torch, taco, synth, base, block, steps, warmup, use_graph,
                         packed=kind == "owner_packed")
    elif kind == "packed":
        res = packed_case(torch, taco, synth, base, block, steps, warmup, use_graph)
    elif kind == "accn":
        res = accumulate_case(torch, taco, synth, base, block, steps, warmup, use_graph,
                              fused=True)
    elif kind == "fidelity":
        res = fidelity_case(torch, taco, synth, base, block, steps, warmup, use_graph)
    elif kind in ("e5m2", "int8"):
        res = roundtrip_case(torch, taco, synth, base, block, steps, warmup, use_graph, kind)
    elif kind:
        raise SystemExit(f"unknown workload variant {name!r}")
    elif acc:
        res = accumulate_case(torch, taco, synth, base, block, steps, warmup, use_graph,
                              also_fused=also_fused)
    else:
        res = roundtrip_case(torch, taco, synth, base, block, steps, warmup, use_graph)
    torch.cuda.empty_cache()
    return res, base, acc


def same_mix_reference(torch, res, use_graph: bool) -> dict:
    """A plain stream with compress's byte mix at the same size, measured in
    the same run (context for the roofline)."""
    ref = add_reference(torch, res["n"], use_graph)
    ref["kernel"] = "torch.add, bf16, reads 2N bytes and writes N (the compress byte mix)"
    ref["compress_rate_vs_reference"] = round((ref["us"] * 1e-6) / res["kernels"]["compress"], 4)
    return ref


def add_floors(torch, rec: dict, res: dict, use_graph: bool) -> None:
    """roofline.launch_floor and roofline.stream_floor for the line's
    dominant kernel (compress, decompress or accumulate), measured in the
    same run."""
    import gradients_taco_compress_amd.probe as probe
    roof = rec["roofline"]
    kern = roof["kernel"]
    if kern not in ("compress", "decompress", "accumulate"):
        return
    print("[bench] launch and stream floors (libtaco_probe)", file=sys.stderr, flush=True)
    n, block = res["n"], res["block"]
    roof["launch_floor"] = launch_floor(torch, probe, launch_groups(n, block), use_graph)
    roof["stream_floor"] = stream_floor(torch, probe, kern, n, roof["algorithmic_bytes"],
                                        res["kernels"][kern], use_graph)
    valu = roof.get("valu", {}).get("wave_instructions")
    if valu:
        # The same stream carrying the kernel's own VALU work: its committed
        # SQ_INSTS_VALU count per launch spread over the stream's
        # wavefronts (one per 1024 elements), to a multiple of 4.
        per_wave = max(4, int(round(valu / max(1, n // 1024) / 4.0)) * 4)
        roof["stream_valu_floor"] = stream_floor(torch, probe, kern, n, roof["algorithmic_bytes"],
                                                 res["kernels"][kern], use_graph, per_wave)


def config_summary(rec: dict) -> dict:
    """The figures of one round-trip workload for the default line's
    "configs" list (never part of its value)."""
    out = {"workload": rec["config"]["workload"], "block": rec["config"]["block"],
           "step": rec["config"]["step"], "steps": rec["steps"], "warmup": rec["warmup"],
           "ms_per_step": rec["ms_per_step"], "input_GBps": rec["value"],
           "pct_hbm_peak": rec["pct_hbm_peak"], "kernel_us": rec["kernel_us"],
           "repeats_pct_hbm_peak_median": (rec.get("repeats") or {}).get("pct_hbm_peak_median")}
    roof = rec["roofline"]
    out["roofline"] = {k: roof.get(k) for k in ("kernel", "achieved", "frac", "traffic")}
    for key in ("same_mix_stream", "launch_floor", "stream_floor", "stream_valu_floor"):
        if key in roof:
            out[key] = roof[key]
    return out


def main():
    args = parse()
    if args.steps is not None:
        if args.steps < 1:
            print("--steps must be at least 1", file=sys.stderr)
            sys.exit(2)
    if args.warmup is not None and args.warmup < 0:
        print("--warmup must be at least 0", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the operator "
              "runs on one GPU; sharding is a design, not code here).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(torch)
        return
    import gradients_taco_compress_amd as taco
    import synth

    use_graph = not args.no_graph
    if args.torch_reference:
        names = [args.workload] if args.workload else [
            "laplace_2048x1024", "gpt2.7b_rowpar_8192x2560", "qwen7b_act_16384x3584",
            "grad_8192x8192", "gpt175b_hidden_32768x12288"]
        torch_reference(torch, synth, [(nm, None) for nm in names], use_graph)
        return
    if args.all:
        cases = [("gpt175b_hidden_32768x12288", 256)] + ROUNDTRIP_CONFIGS + [
                 ("gpt175b_hidden_32768x12288:owner", 256),
                 ("gpt175b_hidden_32768x12288:owner_packed", 256),
                 ("gpt175b_hidden_32768x12288:accn", 256),
                 ("gpt2.7b_rowpar_8192x2560:packed", 128),
                 ("gpt2.7b_rowpar_8192x2560:e5m2", 128),
                 ("gpt2.7b_rowpar_8192x2560:int8", 128),
                 ("gpt2.7b_rowpar_8192x2560:fidelity", 128)]
    else:
        name = args.workload or synth.DEFAULT_WORKLOAD
        block = args.block or synth.WORKLOADS[name.split(":")[0]].blocks[0]
        cases = [(name, block)]
    default_line = not args.all and args.workload is None and args.block is None
    recs = []
    for i, (name, block) in enumerate(cases):
        print(f"[bench] {name} block {block}", file=sys.stderr, flush=True)
        res, base, acc = run_case(torch, taco, synth, name, block, args.steps, args.warmup,
                                  use_graph, also_fused=default_line and not args.no_configs)
        cpu = None
        if not args.no_cpu_baseline and i == 0:
            print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
            cpu = cpu_baseline(synth, base, block, args.cpu_seconds, acc)
        rec = record(res, base, args, cpu)
        if "fused_receive" in res:
            rec["fused_receive"] = res["fused_receive"]
        if not args.no_floors and rec["roofline"]["kernel"] == "compress" and \
                not res.get("packed") and (i == 0 or (base, block) in ROUNDTRIP_CONFIGS):
            print("[bench] same-mix stream reference (torch add)", file=sys.stderr, flush=True)
            rec["roofline"]["same_mix_stream"] = same_mix_reference(torch, res, use_graph)
        if i == 0 and not name.split(":")[1:] and not args.no_floors:
            add_floors(torch, rec, res, use_graph)
        recs.append(rec)
        if args.all:
            print(json.dumps(rec), file=sys.stderr, flush=True)
    if default_line and not args.no_configs:
        # The other workloads' round trips, after the default line's timed
        # region: reported beside it, never in its value.
        configs = []
        for name, block in ROUNDTRIP_CONFIGS:
            print(f"[bench] config {name} block {block}", file=sys.stderr, flush=True)
            res, base, _ = run_case(torch, taco, synth, name, block, None, None, use_graph)
            rec = record(res, base, args)
            if not args.no_floors:
                rec["roofline"]["same_mix_stream"] = same_mix_reference(torch, res, use_graph)
                add_floors(torch, rec, res, use_graph)
            configs.append(config_summary(rec))
        recs[0]["configs"] = configs
    if args.out:
        with open(args.out, "w") as f:
            json.dump(recs if args.all else recs[0], f, indent=1)
    print(json.dumps(recs[0]), flush=True)


if __name__ == "__main__":
    main()
