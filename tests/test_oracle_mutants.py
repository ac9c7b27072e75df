"""Planted mistakes in the oracle must each fail the pin suite.

Every case copies the oracle's C source, plants one plausible slip (a
dropped term, an off-by-one set boundary, a wrong head mapping, a
transposed operand, a wrong sign, a missing normalisation or square root),
builds the copy into a temporary library and runs tests/test_oracle_pins.py
against it in a subprocess.  The suite has to fail for every mutant; the
unmodified source has to pass.  All of this runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "alspec_oracle.c")

MUTANTS = {
    "drop_sink_from_set": ("for (int j = 0; j < s_end; ++j) tok_A[nA++] = j;",
                           ""),
    "window_off_by_one": ("int wb = L - W;", "int wb = L - W + 1;"),
    "sink_off_by_one": ("int se = S < L ? S : L;",
                        "int se = S < L ? (S > 0 ? S - 1 : 0) : L;"),
    "gqa_mapping_modulo": ("int g = h / G;", "int g = h % J->Hkv;"),
    "no_renormalisation": ("J->o_approx[o + d] = acc_a[d] / l_a;",
                           "J->o_approx[o + d] = acc_a[d] * exp(m_a - m_e) / l_e;"),
    "values_as_keys": ("dot += (double)q[d] * wk(k, row + (size_t)d);",
                       "dot += (double)q[d] * wk(v, row + (size_t)d);"),
    "wrong_sign_exp": ("double w = exp(s_buf[t] - m);",
                       "double w = exp(m - s_buf[t]);"),
    "scale_dropped": ("double s = sm_scale * dot;", "double s = dot;"),
    "ratio_without_sqrt": ("r = sqrt(num / den);", "r = num / den;"),
    "strict_threshold": ("(uint8_t)(r <= lambda)", "(uint8_t)(r < lambda)"),
    "merge_ignores_shift": ("Z += l[i] * w;", "Z += l[i];"),
    "norm_without_den": ("den += e * e;", "den += 1.0;"),
}


def _build(tmp_path, text, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(text)
    subprocess.run(["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L",
                    "-ffp-contract=off", "-fPIC", "-shared", "-o", str(so),
                    str(c), "-lm", "-lpthread"], check=True)
    return str(so)


def _run_pins(lib):
    env = dict(os.environ, ALSPEC_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                        "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_source_passes(tmp_path):
    lib = _build(tmp_path, open(SRC).read(), "clean")
    rc, out = _run_pins(lib)
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build(tmp_path, text.replace(old, new), name)
    rc, out = _run_pins(lib)
    assert rc != 0, f"pins did not catch mutant {name}:\n{out}"
