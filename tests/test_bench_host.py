"""Host-side logic of bench.py (no GPU): the algorithmic byte counts that the
roofline divides by, the buffer rotation that keeps loads out of the 256 MB
Infinity Cache, the warmup sizing, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("block", [32, 64, 128, 256, 512])
def test_algorithmic_bytes_per_element(block):
    # Per element: bf16 2 bytes, code 1 byte, two float32 scalars per block,
    # float32 accumulator read and written.
    n = block * 1000
    per = 8.0 / block
    assert bench.algorithmic_bytes("compress", n, block) == pytest.approx(n * (3 + per))
    assert bench.algorithmic_bytes("decompress", n, block) == pytest.approx(n * (3 + per))
    assert bench.algorithmic_bytes("accumulate", n, block) == pytest.approx(n * (9 + per))
    for p in (1, 3, 8):
        assert bench.algorithmic_bytes(f"accumulate_n:{p}", n, block) == pytest.approx(
            n * (p * (1 + per) + 8))
        assert bench.algorithmic_bytes(f"reduce_compress:{p}", n, block) == pytest.approx(
            n * (2 + p * (1 + per) + 1 + per))
    with pytest.raises(ValueError):
        bench.algorithmic_bytes("nothing", n, block)


def test_rotation_covers_four_times_the_infinity_cache():
    assert bench.ROTATE_LOAD_BYTES >= 4 * bench.MALL_BYTES
    for load in (4 << 20, 40 << 20, 700 << 20, 3 << 30):
        k = bench.rotation_sets(load, 3 * load)
        assert k >= 1
        capped = -(-bench.ROTATE_LOAD_BYTES // load) * 3 * load > bench.MAX_SET_BYTES
        if not capped:
            assert k * load >= bench.ROTATE_LOAD_BYTES       # loads leave the cache
        assert k == 1 or k * 3 * load <= bench.MAX_SET_BYTES  # and fit the memory cap


def test_default_warmup_moves_enough_bytes_and_covers_every_set():
    step = 128.45e6                                  # the 40 MiB round trip
    w = bench.warmup_steps(None, 49, step)
    assert w >= 49 and w * step >= bench.WARM_BYTES
    assert bench.warmup_steps(None, 500, 1e12) == 500
    assert bench.warmup_steps(None, 1, 1e12) == 20
    assert bench.warmup_steps(7, 49, step) == 7     # an explicit count is kept
    assert bench.warmup_steps(0, 49, step) == 0


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


class _Args:
    warmup = None
    no_graph = False


def _res(kind):
    n, block = 8192 * 2560, 128
    base = {"n": n, "block": block, "steps": 400, "warmup": 779, "sets": 49, "rows": 8192,
            "cols": 2560, "input_bytes_step": 2.0 * n}
    if kind == "roundtrip":
        base.update(t_step=25e-6, kernels={"compress": 12.8e-6, "decompress": 12.5e-6},
                    bytes_step=bench.algorithmic_bytes("compress", n, block)
                    + bench.algorithmic_bytes("decompress", n, block))
    else:
        base.update(t_step=22.9e-6, kernels={"roundtrip": 22.9e-6}, fidelity=True,
                    bytes_step=2.0 * n)
    return base


def test_record_roofline_objects():
    rec = bench.record(_res("roundtrip"), "gpt2.7b_rowpar_8192x2560", _Args())
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["kernel"] == "compress"
    assert roof["achieved"] == pytest.approx(
        bench.algorithmic_bytes("compress", 8192 * 2560, 128) / 12.8e-6 / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / bench.HBM_PEAK_GBS, rel=1e-3)
    if "valu" in roof:        # counters taken on the current kernel source
        v = roof["valu"]
        assert v["bound"] == "alu" and 0 < v["frac"] < 1
        assert v["peak"] == pytest.approx(256 * 4 * 16 * 2.4e9 / 1e12, rel=1e-3)
    fid = bench.record(_res("fidelity"), "gpt2.7b_rowpar_8192x2560", _Args())["roofline"]
    assert fid["bound"] == "alu" and fid["kernel"] == "roundtrip"
    assert fid["hbm"]["frac"] == pytest.approx(2.0 * 8192 * 2560 / 22.9e-6 / 8e12, rel=1e-3)


def test_repeat_stats():
    res = _res("roundtrip")
    assert bench.repeat_stats(res) is None
    res["repeats"] = [25e-6, 26e-6, 24e-6, 30e-6]
    st = bench.repeat_stats(res)
    assert st["n"] == 4 and st["ms_per_step_min"] == 0.024 and st["ms_per_step_max"] == 0.03
    assert st["ms_per_step_median"] == pytest.approx(0.0255)
    assert st["pct_hbm_peak_median"] == pytest.approx(
        100 * res["bytes_step"] / 25.5e-6 / 1e9 / bench.HBM_PEAK_GBS, abs=0.01)


def test_default_line_is_the_largest_workload():
    """The default line times the four-payload X[32768,12288] workload at
    B = 256, and reports the round-trip workloads beside it."""
    import synth
    assert synth.DEFAULT_WORKLOAD == "gpt175b_hidden_32768x12288"
    assert synth.WORKLOADS[synth.DEFAULT_WORKLOAD].blocks[0] == 256
    assert max(w.numel for w in synth.WORKLOADS.values()) == \
        synth.WORKLOADS[synth.DEFAULT_WORKLOAD].numel
    names = {(n, b) for n, b in bench.ROUNDTRIP_CONFIGS}
    for name, w in synth.WORKLOADS.items():
        if name != synth.DEFAULT_WORKLOAD:
            assert {(name, b) for b in w.blocks} <= names


@pytest.mark.parametrize("flag,value", [("--steps", "0"), ("--warmup", "-1")])
def test_bad_step_counts_are_refused(flag, value):
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), flag, value],
                         capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 2 and out.stdout == ""


def test_launch_groups_follow_the_kernels_launch_shape():
    # B = 128 and 256: 8 blocks per wave-step, four wave-steps per group.
    assert bench.launch_groups(8192 * 2560, 128) == 8192 * 2560 // 128 // 8 // 4
    assert bench.launch_groups(2048 * 1024, 128) == 512
    assert bench.launch_groups(8192 * 8192, 256) == 8192 * 8192 // 256 // 8 // 4
    # B = 512: 4 blocks per wave-step; B = 32: 16 blocks, paired from 16384 steps.
    assert bench.launch_groups(512 * 4 * 4 * 10, 512) == 10
    assert bench.launch_groups(32 * 16 * 16383, 32) == -(-16383 // 4)
    assert bench.launch_groups(32 * 16 * 16384, 32) == 16384 // 2 // 4


def test_kernel_hash_covers_exactly_libtaco_sources():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_b", os.path.join(ROOT, "gradients_taco_compress_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    assert sorted(os.path.basename(f) for f in b.ALL_FILES) == sorted(bench.LIBTACO_SOURCES)


def test_kernel_hash_follows_the_build_flags(monkeypatch):
    """The same sources built with other flags are other code: the hash, and
    with it the committed counter runs, change with build.py's FLAGS."""
    h0 = bench.kernel_hash()
    flags = bench.build_flags()
    assert "-amdgpu-kernarg-preload-count=16" in flags and "-packed-fp32-ops" in flags
    monkeypatch.setattr(bench, "build_flags", lambda: flags[:-2])
    assert bench.kernel_hash() != h0


def test_config_summary_carries_the_floors():
    rec = bench.record(_res("roundtrip"), "gpt2.7b_rowpar_8192x2560", _Args())
    rec["roofline"]["launch_floor"] = {"kernel": "empty", "groups": 5120, "us": 2.1}
    rec["roofline"]["stream_floor"] = {"us": 11.2, "frac": 0.70}
    rec["roofline"]["stream_valu_floor"] = {"us": 13.4}
    out = bench.config_summary(rec)
    assert out["workload"] == "gpt2.7b_rowpar_8192x2560" and out["block"] == 128
    assert out["pct_hbm_peak"] == rec["pct_hbm_peak"] and out["input_GBps"] == rec["value"]
    for key in ("launch_floor", "stream_floor", "stream_valu_floor"):
        assert out[key] == rec["roofline"][key]
    assert out["roofline"]["kernel"] == "compress"
