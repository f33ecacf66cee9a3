"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/test_abi.py (validation, the quantizer, block packing, the rotary
table) and tests/test_gguf.py (the GGUF reader on written, truncated and
corrupted files) run again, in a child process, against the sanitized build
(`python -m vision_transformer_amd.build --sanitize`, which the package's
build entry also makes).  Any report aborts the child.  CPU only."""
import os
import subprocess
import sys

import pytest

from vision_transformer_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_is_clean_under_asan_and_ubsan():
    if not os.path.exists(B.SAN_LIB):
        pytest.skip("sanitized library not built (python -m vision_transformer_amd.build --sanitize)")
    if os.path.exists(B.LIB) and os.path.getmtime(B.SAN_LIB) < os.path.getmtime(B.LIB):
        pytest.fail("the sanitized library is older than the main one: rebuild both "
                    "(python -m vision_transformer_amd.build && python -m vision_transformer_amd.build --sanitize)")
    rt = B.sanitizer_runtime()
    if not rt:
        pytest.skip("no sanitizer runtime beside hipcc")
    env = dict(os.environ, JEPA_LIB_PATH=B.SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_gguf.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
