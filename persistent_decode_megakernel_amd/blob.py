"""Read and re-serialise frozen schedule blobs (the layout defined in csrc/sched/layout.h).

Used to inspect schedules and, in tests, to build adversarial mutants for the validator."""
from __future__ import annotations

import ctypes as C
from typing import List

import numpy as np

T_GEMV, T_ATTN, T_ARGMAX = 1, 2, 3
M_QKV, M_O, M_GU, M_D, M_LM = 0, 1, 2, 3, 4

TASK_DTYPE = np.dtype([("type", "u1"), ("mat", "u1"), ("layer", "<u2"), ("id", "<u4"),
                       ("a0", "<u4"), ("a1", "<u4"), ("w0_lo", "<u4"), ("w0_hi", "<u4"),
                       ("w1_lo", "<u4"), ("w1_hi", "<u4"), ("aux0", "<u4"), ("aux1", "<u4"),
                       ("aux2", "<u4"), ("aux3", "<u4")])
assert TASK_DTYPE.itemsize == 48


class BlobConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads",
                                         "head_dim", "ffn", "vocab")] + \
               [("rms_eps", C.c_float), ("rope_theta", C.c_float)] + \
               [(n, C.c_int32) for n in ("tied_lm_head", "wtype", "max_batch", "max_seq",
                                         "group_size")]


class BlobHeader(C.Structure):
    _fields_ = [(n, C.c_uint32) for n in ("magic", "version", "n_cu", "n_tasks", "batch",
                                          "attn_blocks", "n_lm_tiles", "lds_bytes", "ctx_hint",
                                          "placement", "offsets_off", "tasks_off", "total_bytes",
                                          "rotate")] + \
               [("cfg", BlobConfig), ("predicted_us", C.c_double)]


class Blob:
    def __init__(self, data: bytes):
        self.hdr = BlobHeader.from_buffer_copy(data[:C.sizeof(BlobHeader)])
        h = self.hdr
        off = np.frombuffer(data, dtype="<u4", count=h.n_cu + 1, offset=h.offsets_off)
        tasks = np.frombuffer(data, dtype=TASK_DTYPE, count=h.n_tasks, offset=h.tasks_off)
        self.per_cu: List[np.ndarray] = [tasks[off[c]:off[c + 1]].copy() for c in range(h.n_cu)]

    @property
    def n_tasks(self) -> int:
        return sum(len(v) for v in self.per_cu)

    def all_tasks(self) -> np.ndarray:
        return np.concatenate(self.per_cu) if self.per_cu else np.zeros(0, TASK_DTYPE)

    def to_bytes(self) -> bytes:
        h = BlobHeader.from_buffer_copy(bytes(self.hdr))
        n_cu = len(self.per_cu)
        h.n_cu = n_cu
        h.n_tasks = self.n_tasks
        h.offsets_off = C.sizeof(BlobHeader)
        h.tasks_off = (h.offsets_off + 4 * (n_cu + 1) + 63) & ~63
        h.total_bytes = h.tasks_off + TASK_DTYPE.itemsize * h.n_tasks
        out = bytearray(h.total_bytes)
        out[:C.sizeof(h)] = bytes(h)
        offs = np.zeros(n_cu + 1, "<u4")
        k = 0
        for c, v in enumerate(self.per_cu):
            offs[c] = k
            k += len(v)
        offs[n_cu] = k
        out[h.offsets_off:h.offsets_off + 4 * (n_cu + 1)] = offs.tobytes()
        if k:
            out[h.tasks_off:] = self.all_tasks().tobytes()
        return bytes(out)
