"""Build libamk.so in-tree with hipcc for gfx950 (also usable as `python -m ...build`).

Every HIP source is compiled with packed-FP32 instructions disabled. The host-only schedule layer
is plain C++ compiled into the same library."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libamk.so")
BUILD = os.path.join(ROOT, "_build")

HIP_SOURCES = ["kernels/megakernel.hip", "kernels/unfused.hip", "runtime/model.hip"]
CXX_SOURCES = ["runtime/errors.cpp", "sched/builder.cpp", "sched/validate.cpp", "sched/sched_api.cpp",
               "sched/rebalance.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"] + inc
    objs, cmds = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
        cmds.append([hipcc(), f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                     "-packed-fp32-ops", "-c", os.path.join(CSRC, src), "-o", obj] + common)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
        cmds.append(["g++", "-c", os.path.join(CSRC, src), "-o", obj] + common)
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
