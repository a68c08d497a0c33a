"""Planted mistakes: each must make the oracle's own pins fail.

Every case below copies ``oracle/taco_oracle.c``, changes one spot in the
way a plausible slip would (a sign, an index, a dropped term or factor, a
swapped operand, the wrong decoder), builds the copy with the oracle's own
flags, and runs the oracle test files against it (``TACO_ORACLE_MUTANT``)
in a child process: at least one pin must fail.  A control build of the
unchanged source must pass the same run.  The exhaustive 2^32-pattern
encoder checks are left out of these runs for time; every mistake below is
caught without them.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "taco_oracle.c")
PIN_FILES = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py")
                   and f != "test_oracle_mutants.py")

# (name, text in taco_oracle.c, replacement): the text must occur exactly once.
MUTANTS = [
    # Hadamard (Eq. 8 / 12)
    ("fwht_butterfly_sign", "v[j + h] = a - b;", "v[j + h] = b - a;"),
    ("fwht_last_stage_dropped", "for (int h = 1; h < n; h *= 2)",
     "for (int h = 1; h < n / 2; h *= 2)"),
    # Eq. 6-7
    ("energy_not_averaged", "double sigma = sqrt(energy / B + eps);",
     "double sigma = sqrt(energy + eps);"),
    ("eps_outside_root", "double sigma = sqrt(energy / B + eps);",
     "double sigma = sqrt(energy / B) + eps;"),
    ("alpha_inverted", "double alpha = tau / sigma;", "double alpha = tau * sigma;"),
    # Eq. 8-10
    ("forward_not_normalised", "for (int j = 0; j < B; ++j) Z[j] *= c;",
     "for (int j = 0; j < B; ++j) Z[j] *= 1.0;"),
    ("signed_block_max", "zmax = fmax(zmax, fabs(Z[j]));", "zmax = fmax(zmax, Z[j]);"),
    ("scale_off_by_one_qmax", "double s = zmax / taco_oracle_qmax(fmt);",
     "double s = zmax / (taco_oracle_qmax(fmt) - 1.0);"),
    ("quantise_times_scale", "(float)(Z[j] / s)", "(float)(Z[j] * s)"),
    ("zero_keeps_sign", "if (v == 0.0f) v = 0.0f;                   /* zero carries no sign */",
     ";"),
    # Eq. 11-13
    ("dequantise_without_scale", "out[j] = decode_fmt(q[j], fmt) * (double)s;",
     "out[j] = decode_fmt(q[j], fmt);"),
    ("inverse_not_normalised", "out[j] = out[j] * c / (double)alpha; /* Eq. 13 */",
     "out[j] = out[j] / (double)alpha; /* Eq. 13 */"),
    ("alpha_multiplied_back", "out[j] = out[j] * c / (double)alpha; /* Eq. 13 */",
     "out[j] = out[j] * c * (double)alpha; /* Eq. 13 */"),
    # E4M3 codec and rounding
    ("e4m3_bias_8", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3_subnormal_step", "ldexp((double)m, -9) : ldexp(1.0 + m / 8.0",
     "ldexp((double)m, -10) : ldexp(1.0 + m / 8.0"),
    ("ties_round_up", "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    ("e4m3_no_saturation", "if (a >= ORACLE_QMAX) return sign | 0x7E;", ";"),
    ("bf16_truncates", "r = round_half_even(a / step) * step;", "r = floor(a / step) * step;"),
    # receiver reductions and the owner step
    ("accumulate_overwrites", "float gf = (float)g[j];\n            acc[k * B + j] = acc[k * B + j] + gf;",
     "float gf = (float)g[j];\n            acc[k * B + j] = gf;"),
    ("accumulate_n_keeps_last_payload", "for (int j = 0; j < B; ++j) sum[j] += g[j];",
     "for (int j = 0; j < B; ++j) sum[j] = g[j];"),
    ("owner_drops_own_partial",
     "for (int j = 0; j < B; ++j) X[j] = own ? bf16_to_double(own[k * B + j]) : 0.0;",
     "for (int j = 0; j < B; ++j) X[j] = 0.0;"),
    ("owner_subtracts_payloads", "for (int j = 0; j < B; ++j) X[j] += g[j];",
     "for (int j = 0; j < B; ++j) X[j] -= g[j];"),
    # other formats
    ("e5m2_bias_16", "ldexp(1.0 + m / 4.0, e - 15)", "ldexp(1.0 + m / 4.0, e - 16)"),
    ("e5m2_qmax", "#define ORACLE_E5M2_MAX 57344.0", "#define ORACLE_E5M2_MAX 49152.0"),
    ("int8_decoded_unsigned", "return (double)(int8_t)c;", "return (double)c;"),
    ("int8_not_clamped", "double r = (a >= ORACLE_INT8_MAX) ? ORACLE_INT8_MAX : round_half_even(a);",
     "double r = round_half_even(a);"),
    ("receiver_uses_e4m3_decoder", "case ORACLE_FMT_E5M2: return taco_oracle_e5m2_decode(c);",
     "case ORACLE_FMT_E5M2: return taco_oracle_e4m3_decode(c);"),
    # ablation variants and metrics
    ("direct_without_conversion", "ob[j] = decode_fmt(cvt_fmt(G[j], fmt), fmt);", "ob[j] = G[j];"),
    ("ds_signed_max", "for (int j = 0; j < B; ++j) m = fmax(m, fabs(G[j]));",
     "for (int j = 0; j < B; ++j) m = fmax(m, G[j]);"),
    ("ash_without_alpha", "for (int j = 0; j < B; ++j) ob[j] = ob[j] * c / (double)a32;",
     "for (int j = 0; j < B; ++j) ob[j] = ob[j] * c;"),
    ("hadamard_inverse_unscaled", "for (int j = 0; j < B; ++j) ob[j] *= c;",
     "for (int j = 0; j < B; ++j) ob[j] *= 1.0;"),
    ("tensor_scale_from_first_block",
     "for (int64_t i = 0; i < n; ++i) tensor_max = fmax(tensor_max, fabs(bf16_to_double(x[i])));",
     "for (int64_t i = 0; i < B && i < n; ++i) tensor_max = fmax(tensor_max, fabs(bf16_to_double(x[i])));"),
    ("rel_l2_squared", "out[0] = (sr > 0.0) ? sqrt(se) / sqrt(sr) : sqrt(se);",
     "out[0] = (sr > 0.0) ? se / sr : se;"),
    ("cos_without_root", "sd / (sqrt(sg) * sqrt(sr))", "sd / (sg * sr)"),
    ("mse_not_divided", "out[3] = se / (double)n;", "out[3] = se;"),
]


def _build(source: str, out_dir: str, name: str) -> str:
    src = os.path.join(out_dir, name + ".c")
    lib = os.path.join(out_dir, "lib" + name + ".so")
    with open(src, "w") as f:
        f.write(source)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", src, "-o", lib, "-lm"])
    return lib


def _run_pins(lib: str):
    env = dict(os.environ, TACO_ORACLE_MUTANT=lib, PYTHONDONTWRITEBYTECODE="1")
    p = subprocess.run([sys.executable, "-m", "pytest", *PIN_FILES, "-x", "-q",
                        "-k", "not exhaustive", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-2000:] + p.stderr[-2000:]


@pytest.fixture(scope="module")
def results():
    text = open(SRC).read()
    tmp = tempfile.mkdtemp(prefix="taco_mutants_")
    try:
        libs = {"control": _build(text, tmp, "control")}
        for name, old, new in MUTANTS:
            assert text.count(old) == 1, f"{name}: the planted spot must occur exactly once"
            libs[name] = _build(text.replace(old, new), tmp, name)
        workers = max(1, min(8, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(workers) as pool:
            runs = dict(zip(libs, pool.map(_run_pins, libs.values())))
        return runs
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_control_build_passes_the_pins(results):
    rc, out = results["control"]
    assert rc == 0, out


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(results, name):
    rc, out = results[name]
    assert rc == 1 and " failed" in out, f"{name} survived the pins:\n{out}"
