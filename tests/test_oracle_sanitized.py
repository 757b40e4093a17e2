"""The oracle's own pins, re-run against a build of the C oracle compiled with
the address and undefined-behaviour sanitizers (host code only; no GPU).

The sanitized shared object is built into a temporary directory and loaded in
a child interpreter (the ASan runtime has to be the first library of the
process, so it is preloaded there); every sanitizer report aborts that child.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "csa2_oracle.c")
PINS = ["tests/test_oracle_index.py", "tests/test_oracle_attention.py",
        "tests/test_oracle_fp4.py", "tests/test_oracle_block.py", "tests/test_oracle_session.py"]


def _runtime(gcc: str, name: str) -> str:
    path = subprocess.run([gcc, "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    libasan = _runtime(gcc, "libasan.so")
    if not libasan:
        pytest.skip("gcc has no ASan runtime")
    so = str(tmp_path / "libcsa2_oracle_san.so")
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", SRC, "-o", so, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", CSA2_ORACLE_LIB=so,
               PYTHONPATH=ROOT)
    # -s: a sanitizer report ends the child at once, so it must not sit in
    # pytest's capture buffer; no conftest (it would import more than the pins need)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
                        "--noconftest", *PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    report = (r.stdout + r.stderr)[-4000:]
    assert "Sanitizer" not in report and "runtime error" not in report, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
