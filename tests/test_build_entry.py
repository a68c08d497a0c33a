"""The build step must work in a fresh checkout, where libtaco.so does not
exist yet: loading the build module may not import the package (whose
import refuses to proceed without the library)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_module_loads_without_the_package():
    code = ("import sys; sys.path.insert(0, %r); import __graft_entry__ as g; "
            "m = g._load_hip_build(); "
            "assert 'gradients_taco_compress_amd' not in sys.modules; "
            "assert callable(m.build) and m.LIB.endswith('libtaco.so'); print('ok')" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd="/")
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "ok"


def test_build_script_runs_as_a_script_without_the_package():
    # Only checks that the script starts (it imports nothing from the package);
    # compiling is what build() does.
    src = open(os.path.join(ROOT, "gradients_taco_compress_amd", "build.py")).read()
    assert "import gradients_taco_compress_amd" not in src
    assert "from gradients_taco_compress_amd" not in src
    assert "from ." not in src


def test_extra_hipcc_flags_come_from_the_environment(monkeypatch):
    import __graft_entry__ as g
    m = g._load_hip_build()
    monkeypatch.delenv("TACO_HIPCC_FLAGS", raising=False)
    assert m.extra_flags() == []
    monkeypatch.setenv("TACO_HIPCC_FLAGS", " -DTACO_WAVES_PER_GROUP=8  -DTACO_MAX_GROUPS=2048 ")
    assert m.extra_flags() == ["-DTACO_WAVES_PER_GROUP=8", "-DTACO_MAX_GROUPS=2048"]


def test_variant_build_goes_to_its_own_path(monkeypatch, tmp_path):
    """build(out=...) compiles the operator's sources with the extra flags and
    links them to that path only: the in-tree libraries are not rebuilt and
    the probe library is left out."""
    import __graft_entry__ as g
    m = g._load_hip_build()
    cmds = []

    def fake_run(cmd, verbose):
        cmds.append(cmd)
        if "-o" in cmd:
            open(cmd[cmd.index("-o") + 1], "wb").close()
    monkeypatch.setattr(m, "_run", fake_run)
    monkeypatch.setenv("TACO_HIPCC_FLAGS", "-DTACO_WAVES_PER_GROUP=8")
    out = str(tmp_path / "libtaco_wpg8.so")
    assert m.build(out=out) == out and os.path.exists(out)
    compiles = [c for c in cmds if "-c" in c]
    links = [c for c in cmds if "-shared" in c]
    assert sorted(c[c.index("-c") + 1] for c in compiles) == sorted(m.SOURCES)
    assert all("-DTACO_WAVES_PER_GROUP=8" in c for c in compiles)
    assert len(links) == 1 and links[0][links[0].index("-o") + 1].startswith(out)
    assert not any(m.LIB in " ".join(c) or m.PROBE_LIB in " ".join(c) for c in cmds)
    assert not [f for f in os.listdir(m.CSRC) if ".tmp" in f]      # objects removed


def test_every_compile_targets_gfx950_without_packed_fp32(monkeypatch, tmp_path):
    """Each hipcc compile of build() (the default build and a variant built
    with --out) targets gfx950 and turns the packed-FP32 feature off, with
    the optimisation level and no sanitizer."""
    import __graft_entry__ as g
    m = g._load_hip_build()
    cmds = []

    def fake_run(cmd, verbose):
        cmds.append(cmd)
        if "-o" in cmd:
            open(cmd[cmd.index("-o") + 1], "wb").close()
    monkeypatch.setattr(m, "_run", fake_run)
    monkeypatch.setattr(m, "LIB", str(tmp_path / "libtaco.so"))
    monkeypatch.setattr(m, "PROBE_LIB", str(tmp_path / "libtaco_probe.so"))
    monkeypatch.delenv("TACO_HIPCC_FLAGS", raising=False)
    m.build()
    m.build(out=str(tmp_path / "variant.so"))
    compiles = [c for c in cmds if "-c" in c]
    assert len(compiles) == 2 * len(m.SOURCES) + 1            # the probe in the default build
    feature = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    for c in compiles:
        assert "--offload-arch=gfx950" in c and "-O3" in c
        assert any(c[i:i + 4] == feature for i in range(len(c) - 3)), c
        assert not any(a.startswith("-fsanitize") for a in c)
