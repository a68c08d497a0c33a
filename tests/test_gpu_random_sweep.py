"""Seeded random parity sweep on the GPU: block sizes, shapes, the five input
distributions (with random seeds), the three code formats, owner steps with
1-8 payloads with and without an own partial, the multi-payload accumulate
and the fidelity round trip's variants, each compared with the oracle
through the same helpers as the other parity tests."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synth
from parity import FLIP_RATE, compare_compress, compare_decompress, compare_reduce
from test_gpu_accumulate_n import check as accumulate_n_check
from test_gpu_fidelity import check_variant

pytestmark = pytest.mark.gpu

# 300 fixed-seed cases by default; TACO_SWEEP_CASES / TACO_SWEEP_SEED run a
# longer sweep or another seed.  TACO_SWEEP_MAX_ROWS raises the row count's
# upper end (default 200), and TACO_SWEEP_PACKED (a probability, default 0)
# also sends cases through the interleaved wire layout; both are drawn from
# a generator of their own, so the default sequence of cases is unchanged.
CASES = int(os.environ.get("TACO_SWEEP_CASES", "300"))
SEED = int(os.environ.get("TACO_SWEEP_SEED", "20261202"))
MAX_ROWS = int(os.environ.get("TACO_SWEEP_MAX_ROWS", "200"))
PACKED = float(os.environ.get("TACO_SWEEP_PACKED", "0"))


def test_random_sweep():
    import torch
    import gradients_taco_compress_amd as taco

    def gpu_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    def gpu(a, shape=None):
        t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return t.reshape(shape) if shape is not None else t

    names = sorted(synth.WORKLOADS)
    rng = np.random.default_rng(SEED)
    extra = np.random.default_rng([SEED, 1])
    flips = {"e4m3": [0, 0], "e5m2": [0, 0], "int8": [0, 0]}
    owners = 0
    for case in range(CASES):
        B = int(rng.choice([32, 64, 128, 256, 512]))
        fmt = str(rng.choice(["e4m3", "e4m3", "e5m2", "int8"]))
        rows = int(rng.integers(1, 200))
        cols = B * int(rng.integers(1, 24))
        name = str(rng.choice(names))
        seed = int(rng.integers(0, 1 << 30))
        owner = rng.random() < 0.4
        P = int(rng.integers(1, 9))
        with_own = rng.random() < 0.8
        accn = rng.random() < 0.1
        variant = str(rng.choice(["taco", "direct", "ds", "ash", "hadamard", "tensor"]))
        study = rng.random() < 0.1
        if MAX_ROWS > 200 and extra.random() < 0.5:
            rows = int(extra.integers(200, MAX_ROWS + 1))
        packed = extra.random() < PACKED
        print(f"[case] sweep {case}: {name} {rows}x{cols} B={B} fmt={fmt} seed={seed}"
              + (f" owner P={P} own={with_own}" if owner else "")
              + (f" accumulate_n P={P}" if accn else "") + (f" roundtrip {variant}" if study else "")
              + (" packed" if packed else ""), flush=True)
        r = synth.WORKLOADS[name].with_shape(rows, cols, seed=seed)
        x = synth.generate(r)
        c, a, s = taco.compress(gpu_bf16(x), block=B, fmt=fmt)
        torch.cuda.synchronize()
        st = compare_compress(x, B, c.cpu().numpy(), a.cpu().numpy(), s.cpu().numpy(), fmt=fmt)
        flips[fmt][0] += st["flips"]
        flips[fmt][1] += st["n"]
        oc, oa, os_ = st.pop("oracle")
        y = taco.decompress(gpu(oc, x.shape), gpu(oa), gpu(os_), block=B, fmt=fmt)
        torch.cuda.synchronize()
        compare_decompress(y.view(torch.int16).cpu().numpy().view(np.uint16), oc, oa, os_, B,
                           fmt=fmt)
        if packed:
            # The interleaved layout: the GPU payload unpacked and compared
            # like the separate buffers, and the oracle's payload decompressed.
            pay = taco.compress_packed(gpu_bf16(x), block=B, fmt=fmt)
            torch.cuda.synchronize()
            pc, pa, ps = oracle.unpack(pay.cpu().numpy(), B)
            stp = compare_compress(x, B, pc, pa, ps, fmt=fmt)
            flips[fmt][0] += stp["flips"]
            flips[fmt][1] += stp["n"]
            yp = taco.decompress_packed(gpu(oracle.pack(oc, oa, os_, B).reshape(-1)), x.shape,
                                        block=B, fmt=fmt)
            torch.cuda.synchronize()
            compare_decompress(yp.view(torch.int16).cpu().numpy().view(np.uint16), oc, oa, os_,
                               B, fmt=fmt)
        if accn:
            xs = [synth.generate(r.with_shape(rows, cols, seed=seed + 100 + p)) for p in range(P)]
            accumulate_n_check(taco, xs, B, (rng.standard_normal(x.size) * 0.01).astype(np.float32),
                               fmt)
        if study:
            check_variant(taco, x, B, variant, fmt)
        if owner:
            pays = [tuple(oracle.compress(synth.generate(r.with_shape(rows, cols, seed=seed + 1 + p)),
                                          B, fmt=fmt)) for p in range(P)]
            own = x if with_own else None
            co, ao, so = taco.reduce_compress(None if own is None else gpu_bf16(own),
                                              [(gpu(pc, x.shape), gpu(pa), gpu(ps))
                                               for pc, pa, ps in pays], block=B, fmt=fmt)
            torch.cuda.synchronize()
            compare_reduce(own, pays, B, co.cpu().numpy(), ao.cpu().numpy(), so.cpu().numpy(),
                           fmt=fmt)
            owners += 1
    print(f"sweep: {CASES} cases ({owners} owner steps), compress flips per format "
          f"(flips, elements): {flips}", flush=True)
    # The contract's rate on the sweep's own compress comparisons, per format.
    for fmt, (f, n) in flips.items():
        assert f <= FLIP_RATE * max(n, 1), f"{fmt}: {f} flips in {n} elements"
