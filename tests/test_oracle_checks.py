"""Checks on the oracle itself (CPU only).

1. Its pins pass with the oracle built under AddressSanitizer and
   UndefinedBehaviorSanitizer (gcc -fsanitize=address,undefined), and the
   sanitizer is live in that setup: an undersized output buffer passed on
   purpose is reported.
2. The tolerance and quantizer pins reject the oracle when one term of a
   composite tolerance or the quantizer's divisor is changed: each mutant is a
   copy of qi4_oracle.c with one substitution, built into a temporary
   directory and loaded through QI4O_LIB in a subprocess that runs the pins."""
import os
import subprocess
import sys

import pytest

from oracle.build import build_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qi4_oracle.c")
PIN_FILES = ["tests/test_oracle_format.py", "tests/test_oracle_linear.py",
             "tests/test_oracle_moe.py", "tests/test_oracle_int8.py",
             "tests/test_oracle_w4a8.py", "tests/test_oracle_tolerance.py"]


def _gcc_lib(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True, check=True).stdout.strip()


def _run(args, env_extra, timeout=600):
    env = dict(os.environ, **env_extra)
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "libqi4_oracle_san.so")
    build_oracle(out=out, sanitize=True)
    env = {"QI4O_LIB": out,
           "LD_PRELOAD": f"{_gcc_lib('libasan.so')}:{_gcc_lib('libubsan.so')}",
           "ASAN_OPTIONS": "detect_leaks=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
    return env


def test_pins_pass_under_address_and_ub_sanitizers(sanitized):
    r = _run(["-m", "pytest", *PIN_FILES, "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"],
             sanitized)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_sanitizer_reports_an_out_of_bounds_write(sanitized):
    """A planted mistake on the CPU: unpack a 4 x 256 matrix into a buffer of
    half its size.  The sanitized oracle must stop with a report."""
    code = ("import ctypes, numpy as np, oracle\n"
            "L = oracle.lib()\n"
            "qw = np.zeros((4, 128), np.uint8)\n"
            "q = np.zeros(512, np.uint8)\n"
            "L.qi4o_unpack(qw.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), 4, 256, 4,\n"
            "              q.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))\n")
    r = _run(["-c", code], sanitized)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]


# (what is changed, text in qi4_oracle.c, replacement)
MUTANTS = [
    ("gate magnitude for up in tol_h",
     "double ag = c * S[t * N + i], au = c * S[t * N + I + i];",
     "double ag = c * S[t * N + I + i], au = c * S[t * N + i];"),
    ("SiLU deviation dropped from tol_h",
     "tol_h[t * I + i] = silu_dev(g, ag) * (fabs(u) + au) + fabs(qi4o_silu(g)) * au;",
     "tol_h[t * I + i] = ag * (fabs(u) + au) + fabs(qi4o_silu(g)) * au;"),
    ("tol_h ten times too large",
     "tol_h[t * I + i] = silu_dev(g, ag) * (fabs(u) + au) + fabs(qi4o_silu(g)) * au;",
     "tol_h[t * I + i] = 10.0 * (silu_dev(g, ag) * (fabs(u) + au) + fabs(qi4o_silu(g)) * au);"),
    ("down projection's own error dropped",
     "a += fabs(w) * (tol_h[i] + c * (fabs(h[i]) + tol_h[i]));",
     "a += fabs(w) * (tol_h[i] + c * tol_h[i]);"),
    ("h error dropped from the down tolerance",
     "a += fabs(w) * (tol_h[i] + c * (fabs(h[i]) + tol_h[i]));",
     "a += fabs(w) * (c * fabs(h[i]));"),
    ("combine-weight error dropped",
     "if (tt) tt[n] += fabs(pj) * A[n] + eps_p * (fabs(y[n]) + A[n]);",
     "if (tt) tt[n] += fabs(pj) * A[n];"),
    ("shared expert's tolerance dropped",
     "                ot[n] += y[n];\n                if (tt) tt[n] += A[n];",
     "                ot[n] += y[n];"),
    ("W4A8 uncertain-decision term dropped",
     "if (unsure[i]) b += fabs(w) * (double)s_h;",
     "if (unsure[i]) b += 0.0;"),
    ("quantizer divisor 14", "qi4o_f64_to_f16((hi - lo) / L)", "qi4o_f64_to_f16((hi - lo) / (L - 1.0))"),
    ("quantizer divisor 16", "qi4o_f64_to_f16((hi - lo) / L)", "qi4o_f64_to_f16((hi - lo) / (L + 1.0))"),
]


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, what, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found once: {what}"
    mutant = tmp_path / "qi4_oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = str(tmp_path / "libqi4_oracle_mutant.so")
    build_oracle(src=str(mutant), out=lib)
    r = _run(["-m", "pytest", "tests/test_oracle_tolerance.py", "-q", "-x", "-p",
              "no:cacheprovider"], {"QI4O_LIB": lib})
    assert r.returncode != 0, f"the pins accepted the mutant '{what}'"
