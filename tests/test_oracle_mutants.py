"""Planted mistakes: each mutant is a copy of the C oracle with one plausible error
(a dropped term, a wrong sign or index, a swapped operand, a wrong gate). The pin
suite in test_oracle_pins.py must fail on every one of them, which shows the pins
constrain every part of the recurrence. The mutants are built and run on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTANTS = {
    "erase_without_alpha": ("beta * (vr - alpha * sk_dot)", "beta * (vr - sk_dot)"),
    "write_sign_flipped": ("Sr[j] = alpha * Sr[j] + d * kn[j];", "Sr[j] = alpha * Sr[j] - d * kn[j];"),
    "state_not_decayed": ("Sr[j] = alpha * Sr[j] + d * kn[j];", "Sr[j] = Sr[j] + d * kn[j];"),
    "read_before_write": ("Sr[j] = alpha * Sr[j] + d * kn[j];\n        o += Sr[j] * qn[j];",
                          "o += Sr[j] * qn[j];\n        Sr[j] = alpha * Sr[j] + d * kn[j];"),
    "erase_uses_query": ("sk_dot += Sr[j] * kn[j];", "sk_dot += Sr[j] * qn[j];"),
    "query_not_normalised": ("qn[j] *= rq;", "qn[j] *= 1.0;"),
    "key_not_normalised": ("kn[j] *= rk;", "kn[j] *= 1.0;"),
    "head_map_modulo": ("const int h = hv / (HV / H);", "const int h = hv % H;"),
    "beta_sign": ("*beta = 1.0 / (1.0 + exp(-b));", "*beta = 1.0 / (1.0 + exp(b));"),
    "softplus_as_relu": ("(x > 0 ? x : 0.0) + log1p(exp(-fabs(x)))", "(x > 0 ? x : 0.0)"),
    "A_log_not_exponentiated": ("-exp(A_log) * softplus_d(", "-A_log * softplus_d("),
    "dt_bias_dropped": ("softplus_d(a + dt_bias)", "softplus_d(a)"),
    "value_row_index": ("(t * HV + hv) * (int64_t)dv + r)", "(t * HV + hv) * (int64_t)dv + (r + 1) % dv)"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)       # the fp64 loop comes first in the file
    msrc = tmp_path / "gdn_oracle.c"
    msrc.write_text(mutated)
    hdr = os.path.join(ROOT, "oracle", "gdn_oracle.h")
    (tmp_path / "gdn_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(so),
                           str(msrc), "-lm"])
    env = dict(os.environ, GDN_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
