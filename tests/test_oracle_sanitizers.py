"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_driver.c calls every oracle entry point on small
inputs with buffers of exactly the size each call may touch; built with
-fsanitize=address,undefined (recovery off), any out-of-bounds access, use
after free, leak or undefined behaviour in oracle/qlin_oracle.c fails the
run. A standalone executable, so the sanitizer runtimes are linked in and
nothing is preloaded."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_driver")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas",
           os.path.join(ROOT, "oracle", "qlin_oracle.c"), os.path.join(HERE, "sanitize", "oracle_driver.c"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "sanitize" in r.stderr and "unrecognized" in r.stderr:
        pytest.skip("this gcc has no address/undefined sanitizer")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    # the process may already have other libraries preloaded; the sanitizer
    # runtime is linked into the executable, so only its link-order check is relaxed
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all entry points ran" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
