"""The C oracle and the host model of the envelope kernels (both metrics) built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host code only)
and run on random cases: no memory error, no undefined behaviour, and the
drivers' own agreement checks pass (tests/sanitize/*)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, exe, tmp):
    subprocess.run(cmd, check=True, cwd=tmp)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ERROR" not in res.stderr and "runtime error" not in res.stderr, res.stderr
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", *SAN, "-std=c11", "-o", exe, os.path.join(HERE, "sanitize", "oracle_driver.c"),
                os.path.join(ROOT, "oracle", "oracle_edt.c"), "-lm"], exe, tmp_path)
    assert "0 disagreements" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ needed")
def test_host_model_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_model_driver")
    out = _run(["g++", *SAN, "-std=c++17", "-o", exe, os.path.join(HERE, "sanitize", "host_model_driver.cpp")],
               exe, tmp_path)
    assert "0 disagreements" in out
