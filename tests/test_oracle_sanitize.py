"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only), driven over every one of its functions on small inputs
by tests/oracle_sanitize_driver.c.  A sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    src = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    drv = os.path.join(HERE, "oracle_sanitize_driver.c")
    exe = str(tmp_path / "oracle_sanitized")
    flags = [f for f in oracle.CFLAGS if f not in ("-fPIC", "-shared")]
    cmd = ["gcc", *flags, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.dirname(src), "-o", exe, drv, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    # the same flags do catch a heap overflow (the sanitizers are really on)
    bad = tmp_path / "overflow.c"
    bad.write_text("#include <stdlib.h>\nint main(void) { volatile char *p = malloc(8); "
                   "p[8] = 1; free((void *)p); return 0; }\n")
    subprocess.run(["gcc", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", str(tmp_path / "overflow"), str(bad)], check=True, capture_output=True)
    r = subprocess.run([str(tmp_path / "overflow")], capture_output=True, text=True, env=env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
