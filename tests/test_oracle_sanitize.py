"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

``oracle_sanitize_main.c`` calls every oracle entry point on small ragged
shapes with several threads and checks closed forms of the results; here it
is compiled together with ``oracle/mate_oracle.c`` under
``-fsanitize=address,undefined`` (host code only, gcc) and run. Any
out-of-bounds access, use after free, leak, signed overflow or other undefined
behaviour aborts the run.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "tests", "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "mate_oracle.c")]


def test_oracle_under_address_and_ub_sanitizers():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitized")
        flags = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=all", "-pthread"]
        build = subprocess.run([gcc, *flags, *SOURCES, "-o", exe, "-lm"], capture_output=True, text=True)
        if build.returncode != 0 and "asan" in build.stderr.lower():
            pytest.skip("the sanitizer runtime is not installed: " + build.stderr[-300:])
        assert build.returncode == 0, build.stderr
        # verify_asan_link_order=0: the environment may preload other libraries ahead of the runtime
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert run.returncode == 0 and "ALL OK" in run.stdout, run.stdout + run.stderr
