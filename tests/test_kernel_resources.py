"""Resources of the built kernels (host only): the AMDGPU metadata of every gfx950 code object in
libamk.so, read with llvm-readelf. Every batch-1 megakernel instance must run without scratch
memory and without a dynamic stack: a private segment there means a spill or an out-of-line call
(one such build, whose attention staging had become a real call with a 304-byte frame, ended in a
runtime abort on the GPU). The batched instances may spill a few words in their flag polls and
argmax epilogue, never more than a small bound."""
import os
import shutil
import struct
import subprocess
import tempfile

import pytest
import yaml

from persistent_decode_megakernel_amd import _lib

LLVM = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
BATCHED_SPILL_MAX = 64  # bytes per lane


def _code_objects(lib_path: str):
    """The gfx950 code objects of the library's .hip_fatbin section (one offload bundle per
    compiled source, back to back)."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}",
                        lib_path, os.path.join(d, "stripped")], check=True, capture_output=True)
        data = open(fat, "rb").read()
    out = []
    at = data.find(BUNDLE_MAGIC)
    while at >= 0:
        n = struct.unpack_from("<Q", data, at + len(BUNDLE_MAGIC))[0]
        p = at + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            if "gfx950" in triple and size:
                out.append(data[at + off:at + off + size])
        at = data.find(BUNDLE_MAGIC, at + 1)
    return out


def _kernels(code_object: bytes):
    """amdhsa.kernels of one code object's AMDGPU metadata note."""
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(code_object)
        f.flush()
        txt = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", f.name],
                             check=True, capture_output=True, text=True).stdout
    # the document's start and end markers are indented in the listing, its body is not
    lines = txt.splitlines()
    start = next(i for i, l in enumerate(lines) if l.strip() == "---")
    end = next(i for i in range(start + 1, len(lines)) if lines[i].strip() == "...")
    meta = yaml.safe_load("\n".join(lines[start + 1:end]))
    return meta.get("amdhsa.kernels", [])


@pytest.fixture(scope="module")
def kernels(libamk):
    if not os.path.exists(os.path.join(LLVM, "llvm-readelf")) or not shutil.which("python3"):
        pytest.skip("ROCm LLVM tools not found")
    ks = {}
    for co in _code_objects(os.environ.get("AMK_LIB_PATH") or _lib.LIB_PATH):  # the library load() opens
        for k in _kernels(co):
            ks[k[".name"]] = k
    return ks


def test_every_megakernel_instance_is_present(kernels):
    for wt in (0, 1, 2):
        for hd in (64, 128):
            for q in (1, 2, 4):
                for suffix in ("", "_b"):
                    assert f"amk_megakernel_w{wt}_h{hd}_q{q}{suffix}" in kernels


def test_batch1_instances_use_no_scratch(kernels):
    b1 = {n: k for n, k in kernels.items() if n.startswith("amk_megakernel_") and not n.endswith("_b")}
    assert len(b1) == 18
    bad = {n: (k[".private_segment_fixed_size"], k.get(".uses_dynamic_stack", False))
           for n, k in b1.items()
           if k[".private_segment_fixed_size"] != 0 or k.get(".uses_dynamic_stack", False)}
    assert not bad, f"batch-1 instances with scratch or a dynamic stack: {bad}"


def test_batched_instances_spill_little(kernels):
    b = {n: k for n, k in kernels.items() if n.startswith("amk_megakernel_") and n.endswith("_b")}
    assert len(b) == 18
    for n, k in b.items():
        assert not k.get(".uses_dynamic_stack", False), n
        assert k[".private_segment_fixed_size"] <= BATCHED_SPILL_MAX, (n, k[".private_segment_fixed_size"])
