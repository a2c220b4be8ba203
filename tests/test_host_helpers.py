"""Host build of helpers shared with the device code (csrc/sched/layout.h), compiled with g++ and
run: the buffer-address widening that keeps a low address word with bit 31 set from being
sign-extended, the KV-block partition and the packed QKV row map. CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCHED = os.path.join(ROOT, "persistent_decode_megakernel_amd", "csrc", "sched")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_layout_helpers_on_the_host(tmp_path):
    exe = str(tmp_path / "layout_helpers_test")
    src = os.path.join(ROOT, "tests", "host", "layout_helpers_test.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", SCHED, src, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
