"""The oracle's pins run again against a build of the oracle under
AddressSanitizer and UndefinedBehaviorSanitizer (g++ -fsanitize=address,
undefined, errors fatal).  CPU only: the pins run in a child process that
preloads the ASan runtime (the Python interpreter itself is not
instrumented) and loads the sanitized library through SWGQA_ORACLE_LIB.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the layout / brute-force, step-split, rollback, staging-criterion, rotary
# and int8 / fp8 pins: every path of the oracle's forward and plan
PINS = "p2 or p3 or p4 or p10 or p13 or p14 or p15 or invalid or argument"


def _runtime(name: str) -> str:
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    return out.stdout.strip()


def test_pins_pass_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime next to g++")
    lib = oracle.build(force=True, sanitize=True, out=str(tmp_path / "libswgqa_oracle_san.so"))
    env = dict(os.environ)
    env.update(
        SWGQA_ORACLE_LIB=lib,
        LD_PRELOAD=asan,
        # CPython keeps its own arenas alive at exit: leaks are not findings
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
        OMP_NUM_THREADS="4",
    )
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", PINS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert " passed" in r.stdout, tail
