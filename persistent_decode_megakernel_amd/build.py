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

HIP_SOURCES = ["kernels/unfused.hip", "runtime/model.hip", "runtime/calibrate.hip"]
# the megakernel source is compiled once per (weight type, head_dim) pair, in parallel
MEGAKERNEL = "kernels/megakernel.hip"
MK_PAIRS = [(wt, hd) for wt in (0, 1, 2) for hd in (64, 128)]
CXX_SOURCES = ["runtime/errors.cpp", "sched/builder.cpp", "sched/validate.cpp", "sched/sched_api.cpp",
               "sched/rebalance.cpp", "sched/cost_model.cpp", "sched/cost_fit.cpp"]
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


def _headers():
    out = []
    for d in (CSRC, os.path.join(ROOT, "include")):
        for dp, _, fs in os.walk(d):
            out += [os.path.join(dp, f) for f in fs if f.endswith(".h")]
    return out


def _stale(obj: str, src: str, newest_header: float) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return os.path.getmtime(src) > t or newest_header > t


def build(verbose: bool = False, jobs: int = 8, incremental: bool = False) -> str:
    """Compile every source and link libamk.so. incremental=True recompiles only objects older
    than their source or any header (for development loops; the default rebuilds everything)."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"] + inc
    hip = [hipcc(), f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops"]
    newest_header = max((os.path.getmtime(h) for h in _headers()), default=0.0)
    objs, cmds = [], []

    def add(cmd, src, obj):
        objs.append(obj)
        if not incremental or _stale(obj, src, newest_header):
            cmds.append(cmd)

    for wt, hd in MK_PAIRS:
        src = os.path.join(CSRC, MEGAKERNEL)
        obj = os.path.join(BUILD, f"kernels_megakernel_w{wt}_h{hd}.o")
        add(hip + [f"-DAMK_MK_WT={wt}", f"-DAMK_MK_HD={hd}", "-c", src, "-o", obj] + common, src, obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
        add(hip + ["-c", os.path.join(CSRC, src), "-o", obj] + common, os.path.join(CSRC, src), obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
        add(["g++", "-c", os.path.join(CSRC, src), "-o", obj] + common, os.path.join(CSRC, src), obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ["-ldl"])
    os.replace(tmp, OUT)
    return OUT


SANITIZED_OUT = os.path.join(BUILD, "sanitize", "libamk_sched_sanitized.so")


def build_sched_sanitized() -> str:
    """The host-only schedule layer (builder, validator, simulator, re-tiler and their C entry
    points; no HIP code) as a shared library built with AddressSanitizer and UndefinedBehavior-
    Sanitizer, for running the adversarial blob corpus under them. Load it with libasan preloaded
    (the process must start with the ASan runtime) and AMK_LIB_HOST_ONLY=1."""
    os.makedirs(os.path.dirname(SANITIZED_OUT), exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in CXX_SOURCES]
    _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", os.path.join(ROOT, "include"), "-o", SANITIZED_OUT] + srcs + ["-ldl"])
    return SANITIZED_OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
