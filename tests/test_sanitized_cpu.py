"""The fp64 oracle and the input generator built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc), running the oracle's CPU pins in a child
process that loads those builds: an out-of-bounds access, a use after free or
undefined behaviour in either C source fails the pins."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_lib(name):
    p = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _build(src, out):
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared",
                           "-o", out, src, "-lm"])


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_lib("libasan.so"), _gcc_lib("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    synth_so = str(tmp_path / "libsynth_san.so")
    oracle_so = str(tmp_path / "liboracle_san.so")
    _build(os.path.join(ROOT, "synth", "synth.c"), synth_so)
    _build(os.path.join(ROOT, "oracle", "oracle.c"), oracle_so)
    env = dict(os.environ, LM_SYNTH_LIB=synth_so, LM_ORACLE_LIB=oracle_so, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle_pins.py"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=1200)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
