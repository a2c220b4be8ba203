"""The host schedule layer under AddressSanitizer and UndefinedBehaviorSanitizer: the parser,
validator, simulator and re-tiler consume caller-supplied (possibly adversarial) blobs, so the
schedule tests, adversarial corpus and corrupt-blob cases included, run again against a
sanitizer build of that layer in a child process. Any invalid memory access or undefined
behaviour aborts the child. CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if shutil.which("g++") is None:
        return None
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_asan_runtime() is None, reason="g++ with the ASan runtime not available")
def test_schedule_layer_clean_under_asan_and_ubsan():
    from persistent_decode_megakernel_amd import build
    lib = build.build_sched_sanitized()
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), AMK_LIB_PATH=lib, AMK_LIB_HOST_ONLY="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_schedule.py", "tests/test_rebalance.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
