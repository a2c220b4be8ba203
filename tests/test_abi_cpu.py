"""The C ABI library loads on the CPU and exports every symbol include/amk.h declares; argument
errors are reported before any device work (no GPU calls are made here)."""
import ctypes as C
import os
import re

import pytest

from persistent_decode_megakernel_amd import _lib, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "amk.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(amk_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("amk_model_create", "amk_kv_alloc", "amk_decode_step", "amk_destroy"):
        assert n in names


def test_every_declared_symbol_is_exported(libamk):
    for name in declared_functions():
        assert hasattr(libamk, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def test_argument_errors_without_gpu(libamk):
    assert libamk.amk_model_create(None, None, 0, None, 0, None, None) == _lib.AMK_E_INVALID
    assert b"null" in libamk.amk_last_error()
    assert libamk.amk_decode_step(None, None, None, 0, 1, None, None, None) == _lib.AMK_E_INVALID
    assert libamk.amk_kv_bytes(None, 1, 1, None) == _lib.AMK_E_INVALID
    assert libamk.amk_kv_free(None) == _lib.AMK_E_INVALID
    assert libamk.amk_destroy(None) == _lib.AMK_E_INVALID
    assert libamk.amk_sync(None, None) == _lib.AMK_E_INVALID
    assert libamk.amk_decode_steps(None, None, None, 0, 1, 1, None, None, None) == _lib.AMK_E_INVALID
    pos = (C.c_int32 * 2)(0, 0)
    assert libamk.amk_decode_steps_ragged(None, None, None, pos, 1, 2, None, None, None) == _lib.AMK_E_INVALID
    assert libamk.amk_prefill(None, None, 0, None, 0, 1, None, None, None) == _lib.AMK_E_INVALID
    assert b"amk_prefill" in libamk.amk_last_error()
    # invalid config rejected before any device call
    cfg = _lib.make_config(synth.get_config("tiny"))
    cfg.n_heads = 3  # not a multiple of n_kv_heads, hidden != heads * head_dim
    w = _lib.amk_weights()
    out = C.c_void_p()
    assert libamk.amk_model_create(C.byref(cfg), C.byref(w), 0, None, 0, None, C.byref(out)) == _lib.AMK_E_INVALID
    cfg = _lib.make_config(synth.get_config("tiny"))
    cfg.head_dim = 32
    cfg.n_heads = 8
    cfg.n_kv_heads = 4
    assert libamk.amk_model_create(C.byref(cfg), C.byref(w), 0, None, 0, None, C.byref(out)) == _lib.AMK_E_UNSUPPORTED
