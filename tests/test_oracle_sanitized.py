"""The oracle's pins against an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle.c (CPU only).

The pins run in a child process that preloads gcc's sanitizer runtimes and
loads the instrumented library instead of the default build; any invalid
memory access or undefined behaviour in the oracle aborts that process.
"""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(lib, select=None):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    env = dict(os.environ)
    env.update({oracle.LIBRARY_ENV: lib, "LD_PRELOAD": f"{asan}:{ubsan}",
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "OMP_NUM_THREADS": "4"})
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
           "-m", "not gpu", os.path.join(ROOT, "tests", "test_oracle_pins.py")]
    if select:
        cmd += ["-k", select]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=900)


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = oracle.compile_library(str(tmp_path / "liboracle_san.so"), sanitize=True)
    r = _run_pins(lib)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, log
    assert " passed" in r.stdout, log


def test_sanitizer_build_catches_a_planted_overread(tmp_path):
    """Mutant 20 reads one double before its work buffer and changes no
    result: the pins alone cannot see it, the sanitizer build aborts on it."""
    plain = oracle.load_mutant(20, str(tmp_path))
    oracle_pins_mod = __import__("oracle_pins")
    oracle_pins_mod.pin_rho_zero_decode_is_sdpa(oracle.Oracle(plain))
    oracle_pins_mod.pin_single_key(oracle.Oracle(plain))
    lib = oracle.compile_library(str(tmp_path / "liboracle_m20_san.so"), mutant=20,
                                 sanitize=True)
    r = _run_pins(lib, select="rho_zero_decode")
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr, r.stderr[-2000:]
