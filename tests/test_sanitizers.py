"""The oracle and the library's host codebook code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

- The oracle, built with both sanitizers, runs every oracle pin
  (tests/test_oracle_*.py) in a child interpreter that preloads the ASan
  runtime and loads that build instead of the default one.
- The library's codebook builder (codebook.cpp, host code), built with both
  sanitizers together with the sanitized oracle, builds codebooks for a grid
  of models and samples and checks them against the oracle's
  (tests/sanitize_codebook.cpp).
Any sanitizer report fails the test (no recovery; leaks are not checked:
the interpreter itself holds memory to the end).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _asan_runtime():
    p = subprocess.check_output(["gcc", "-print-file-name=libasan.so"]).decode().strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("no ASan runtime for gcc")
    return p


@pytest.mark.slow
def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liblct_oracle_san.so")
    subprocess.check_call(["gcc", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"] + SAN +
                          ["-o", lib, os.path.join(ROOT, "oracle", "lct_oracle.c"), "-lm"])
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), LCT_ORACLE_LIB=lib, **ENV)
    env.pop("PYTEST_XDIST_WORKER", None)
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-p", "no:xdist"]
                       + pins, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out


@pytest.mark.slow
def test_host_codebook_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_codebook")
    ocf = str(tmp_path / "lct_oracle.o")
    subprocess.check_call(["gcc", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-c"] + SAN +
                          ["-o", ocf, os.path.join(ROOT, "oracle", "lct_oracle.c")])
    subprocess.check_call(["g++", "-std=c++17", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include"] + SAN +
                          ["-o", exe, os.path.join(ROOT, "tests", "sanitize_codebook.cpp"),
                           os.path.join(ROOT, "lossless_bf16_tensor_split_amd", "csrc", "codebook.cpp"), ocf, "-lm"])
    r = subprocess.run([exe], env=dict(os.environ, **ENV), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "mismatches: 0" in out
    assert "differing bins: 0" in out and "pmfs checked: 0" not in out
    # the library's Student-t pmf at large nu against 50-digit values of the
    # survival function I_{nu/(nu+u^2)}(nu/2, 1/2) (mpmath's regularized
    # incomplete beta), bin by bin
    import mpmath as mp
    mp.mp.dps = 50
    rows = [ln.split()[1:] for ln in out.splitlines() if ln.startswith("libpmf ")]
    assert len(rows) > 20
    def surv(nu, u):
        return mp.betainc(nu / 2, mp.mpf(1) / 2, 0, nu / (nu + u * u), regularized=True)
    for nu_s, scale_s, e_s, p_s in rows:
        nu, scale, e = mp.mpf(nu_s), mp.mpf(scale_s), int(e_s)
        lo = mp.ldexp(1, e - 127) / scale
        exact = surv(nu, lo) - surv(nu, 2 * lo)
        assert abs(float(p_s) - exact) <= 1e-13 * exact, (nu_s, scale_s, e, p_s, exact)
