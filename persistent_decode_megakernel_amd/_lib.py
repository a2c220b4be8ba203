"""ctypes binding of libamk.so (argument marshalling only; every step of the path runs in the
library's HIP kernels).

The structures below mirror include/amk.h field for field."""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libamk.so")

AMK_OK = 0
AMK_E_INVALID = 1
AMK_E_UNSUPPORTED = 2
AMK_E_OOM = 3
AMK_E_SCHEDULE_REJECTED = 4
AMK_E_HIP = 5
AMK_E_CAPACITY = 6
AMK_E_DEVICE_TIMEOUT = 7
AMK_E_DEVICE_FAULT = 8
AMK_STATIC_SCRATCH_BYTES = 64 << 20  # capacity of the array behind amk_decode_steps_noalloc

AMK_WT_BF16 = 0
AMK_WT_INT8 = 1
AMK_WT_INT4 = 2
AMK_PATH_MEGAKERNEL = 0
AMK_PATH_UNFUSED = 1

STATUS_NAMES = {0: "AMK_OK", 1: "AMK_E_INVALID", 2: "AMK_E_UNSUPPORTED", 3: "AMK_E_OOM",
                4: "AMK_E_SCHEDULE_REJECTED", 5: "AMK_E_HIP", 6: "AMK_E_CAPACITY",
                7: "AMK_E_DEVICE_TIMEOUT", 8: "AMK_E_DEVICE_FAULT"}


class amk_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("tied_lm_head", C.c_int32), ("wtype", C.c_int32), ("max_batch", C.c_int32),
                ("max_seq", C.c_int32), ("group_size", C.c_int32)]


class amk_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")] + \
               [(n, C.c_void_p) for n in ("sq", "sk", "sv", "so", "sg", "su", "sd")] + \
               [("attn_norm", C.c_void_p), ("mlp_norm", C.c_void_p)]


class amk_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("lm_head_scale", C.c_void_p), ("layers", C.POINTER(amk_layer_weights))]


class amk_sched_params(C.Structure):
    _fields_ = [("attn_blocks", C.c_int32), ("min_block", C.c_int32), ("placement", C.c_int32),
                ("rotate", C.c_int32), ("ctx_hint", C.c_int32), ("min_tile_kb", C.c_int32),
                ("search", C.c_int32), ("heads_per_task", C.c_int32)]


class amk_cost_model(C.Structure):
    _fields_ = [("cu_stream_gbs", C.c_double), ("hop_us", C.c_double), ("task_us", C.c_double),
                ("l2_gbs", C.c_double), ("prefetch_kb", C.c_double), ("attn_us", C.c_double)]


class amk_model_info(C.Structure):
    _fields_ = [("n_cu", C.c_int32), ("n_tasks", C.c_int32), ("launches_per_step", C.c_int32),
                ("lds_bytes", C.c_int32), ("attn_blocks", C.c_int32), ("path", C.c_int32),
                ("weight_bytes", C.c_uint64), ("predicted_us", C.c_double),
                ("scratch_bytes", C.c_uint64), ("heads_per_pass", C.c_int32)]


# name -> (restype, argtypes); every symbol include/amk.h declares
SIGNATURES = {
    "amk_model_create": (C.c_int, [C.POINTER(amk_config), C.POINTER(amk_weights), C.c_int32,
                                   C.c_void_p, C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p)]),
    "amk_kv_bytes": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)]),
    "amk_kv_alloc": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_size_t,
                               C.POINTER(C.c_void_p)]),
    "amk_kv_data": (C.c_int, [C.c_void_p, C.POINTER(C.c_void_p)]),
    "amk_decode_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.c_void_p]),
    "amk_decode_steps": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                   C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "amk_decode_steps_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                           C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                           C.c_void_p]),
    "amk_decode_steps_ragged": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(C.c_int32),
                                          C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "amk_prefill": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32,
                              C.c_void_p, C.c_void_p, C.c_void_p]),
    "amk_sync": (C.c_int, [C.c_void_p, C.c_void_p]),
    "amk_model_get_info": (C.c_int, [C.c_void_p, C.POINTER(amk_model_info)]),
    "amk_trace_enable": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t]),
    "amk_model_get_schedule": (C.c_int, [C.c_void_p, C.POINTER(C.c_void_p),
                                         C.POINTER(C.c_size_t)]),
    "amk_model_set_schedule": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "amk_model_tune": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                 C.c_double, C.c_void_p, C.POINTER(C.c_double)]),
    "amk_kv_free": (C.c_int, [C.c_void_p]),
    "amk_destroy": (C.c_int, [C.c_void_p]),
    "amk_last_error": (C.c_char_p, []),
    "amk_schedule_build": (C.c_int, [C.POINTER(amk_config), C.c_int32, C.c_int32,
                                     C.POINTER(amk_sched_params), C.POINTER(amk_cost_model),
                                     C.POINTER(C.c_void_p), C.POINTER(C.c_size_t)]),
    "amk_schedule_validate": (C.c_int, [C.c_void_p, C.c_size_t, C.c_char_p, C.c_size_t]),
    "amk_schedule_simulate": (C.c_int, [C.c_void_p, C.c_size_t, C.c_char_p, C.c_size_t]),
    "amk_schedule_predict": (C.c_int, [C.c_void_p, C.c_size_t, C.POINTER(amk_cost_model),
                                       C.c_int32, C.POINTER(C.c_double)]),
    "amk_schedule_rebalance": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32, C.c_double,
                                         C.POINTER(C.c_void_p), C.POINTER(C.c_size_t)]),
    "amk_calibrate": (C.c_int, [C.POINTER(amk_cost_model), C.c_char_p, C.c_size_t, C.c_void_p]),
    "amk_cost_model_default": (C.c_int, [C.c_int32, C.POINTER(amk_cost_model), C.c_char_p,
                                         C.c_size_t]),
    "amk_schedule_predict_trace": (C.c_int, [C.c_void_p, C.c_size_t, C.POINTER(amk_cost_model),
                                             C.c_int32, C.c_void_p, C.c_size_t]),
    "amk_cost_model_fit": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32, C.c_int32,
                                     C.POINTER(amk_cost_model), C.POINTER(amk_cost_model),
                                     C.c_char_p, C.c_size_t]),
    "amk_blob_free": (None, [C.c_void_p]),
}

_lib: Optional[C.CDLL] = None


class AmkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def load(path: Optional[str] = None) -> C.CDLL:
    """Load libamk.so (built in-tree). Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("AMK_LIB_PATH") or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with persistent_decode_megakernel_amd.build (hipcc, gfx950)")
    lib = C.CDLL(p)
    # AMK_LIB_HOST_ONLY=1: a build of the host schedule layer alone (e.g. the sanitizer build),
    # which exports only the schedule entry points
    host_only = os.environ.get("AMK_LIB_HOST_ONLY") == "1"
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name, None)
        if fn is None:
            if host_only:
                continue
            raise AttributeError(f"{p} does not export {name}")
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(status: int, what: str = "") -> None:
    if status != AMK_OK:
        msg = load().amk_last_error()
        raise AmkError(status, (what + ": " if what else "") + (msg.decode() if msg else ""))


def make_config(cfg, max_batch: Optional[int] = None, max_seq: Optional[int] = None) -> amk_config:
    """amk_config from a synth.Config."""
    return amk_config(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                      cfg.ffn, cfg.vocab, cfg.rms_eps, cfg.rope_theta, int(cfg.tied),
                      {"bf16": AMK_WT_BF16, "int8": AMK_WT_INT8, "int4": AMK_WT_INT4}[cfg.wtype],
                      max_batch or cfg.batch, max_seq or cfg.max_seq,
                      cfg.group if cfg.wtype == "int4" else 0)


def schedule_build(cfg: amk_config, batch: int, n_cu: int,
                   params: Optional[amk_sched_params] = None,
                   cost: Optional[amk_cost_model] = None) -> bytes:
    lib = load()
    blob = C.c_void_p()
    n = C.c_size_t()
    st = lib.amk_schedule_build(C.byref(cfg), batch, n_cu,
                                C.byref(params) if params is not None else None,
                                C.byref(cost) if cost is not None else None,
                                C.byref(blob), C.byref(n))
    check(st, "amk_schedule_build")
    try:
        return C.string_at(blob, n.value)
    finally:
        lib.amk_blob_free(blob)


def schedule_validate(blob: bytes):
    buf = C.create_string_buffer(1024)
    st = load().amk_schedule_validate(blob, len(blob), buf, 1024)
    return st, buf.value.decode()


def schedule_simulate(blob: bytes):
    buf = C.create_string_buffer(1024)
    st = load().amk_schedule_simulate(blob, len(blob), buf, 1024)
    return st, buf.value.decode()


def schedule_predict(blob: bytes, ctx: int, cost: Optional[amk_cost_model] = None) -> float:
    out = C.c_double()
    check(load().amk_schedule_predict(blob, len(blob), C.byref(cost) if cost else None, ctx,
                                      C.byref(out)), "amk_schedule_predict")
    return out.value


def schedule_rebalance(blob: bytes, traces, gain: float = 0.5) -> bytes:
    """Re-tile a schedule from task traces (numpy uint64 array, n_traces x (4 n_tasks + n_cu))."""
    import numpy as np
    lib = load()
    tr = np.ascontiguousarray(traces, dtype=np.uint64)
    n_traces = tr.shape[0] if tr.ndim == 2 else 1
    out = C.c_void_p()
    n = C.c_size_t()
    check(lib.amk_schedule_rebalance(blob, len(blob), tr.ctypes.data_as(C.c_void_p), n_traces,
                                     float(gain), C.byref(out), C.byref(n)),
          "amk_schedule_rebalance")
    try:
        return C.string_at(out, n.value)
    finally:
        lib.amk_blob_free(out)


def schedule_predict_trace(blob: bytes, ctx: int, cost: Optional[amk_cost_model] = None):
    """The cost model's timeline of one step as a task trace (numpy uint64, 4 n_tasks + n_cu)."""
    import numpy as np
    from .blob import Blob
    b = Blob(blob)
    tr = np.zeros(4 * b.hdr.n_tasks + b.hdr.n_cu, dtype=np.uint64)
    check(load().amk_schedule_predict_trace(blob, len(blob), C.byref(cost) if cost else None, ctx,
                                            tr.ctypes.data_as(C.c_void_p), tr.size),
          "amk_schedule_predict_trace")
    return tr


def cost_model_fit(blob: bytes, traces, ctx: int, base: Optional[amk_cost_model] = None):
    """(amk_cost_model fitted to task traces of steps at context ctx, report as a dict)."""
    import json
    import numpy as np
    tr = np.ascontiguousarray(traces, dtype=np.uint64)
    n_traces = tr.shape[0] if tr.ndim == 2 else 1
    out = amk_cost_model()
    buf = C.create_string_buffer(1024)
    check(load().amk_cost_model_fit(blob, len(blob), tr.ctypes.data_as(C.c_void_p), n_traces, ctx,
                                    C.byref(base) if base else None, C.byref(out), buf, len(buf)),
          "amk_cost_model_fit")
    return out, json.loads(buf.value.decode())


def calibrate(stream=None):
    """amk_calibrate on the current device: (fitted amk_cost_model, measurements as a dict)."""
    import json
    cm = amk_cost_model()
    buf = C.create_string_buffer(1 << 16)
    check(load().amk_calibrate(C.byref(cm), buf, len(buf), stream), "amk_calibrate")
    return cm, json.loads(buf.value.decode())


def cost_model_default(n_cu: int):
    """(amk_cost_model the search uses for n_cu CUs when given none, where it came from)."""
    cm = amk_cost_model()
    buf = C.create_string_buffer(4096)
    check(load().amk_cost_model_default(n_cu, C.byref(cm), buf, len(buf)), "amk_cost_model_default")
    return cm, buf.value.decode()
