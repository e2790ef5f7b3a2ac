"""The host side of the library under AddressSanitizer + UndefinedBehaviorSanitizer: the C-ABI
tests (argument validation, status strings, the block KV cache state machine and slot map)
run in a child process against a build whose host code is instrumented, with the sanitizer
runtime preloaded. Any report (an out-of-bounds access, a use after free, signed overflow, an
overlong shift, a misaligned load) ends the child with an error. CPU only."""
import os
import subprocess
import sys

from exact_attention_forward_flash_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _san_lib():
    want = b.source_hash().encode()
    if not (os.path.exists(b.SAN_LIB) and want in open(b.SAN_LIB, "rb").read()):
        b.build(verbose=False, sanitize=True)
    return b.SAN_LIB


def test_abi_suite_under_asan_and_ubsan():
    lib = _san_lib()
    env = dict(os.environ, WF_LIBRARY=lib, LD_PRELOAD=b.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    text = p.stdout + p.stderr
    assert p.returncode == 0, text[-4000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert " passed" in text
