"""Thin Python layer over libamk.so: moves synthetic weights into device memory with torch, calls
the C ABI, and hands back torch tensors. Every step of the decode path runs in the library's HIP
kernels; there is no other implementation here and no fallback."""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from . import _lib
from .synth import MATS, Config, Weights

PATHS = {"megakernel": _lib.AMK_PATH_MEGAKERNEL, "unfused": _lib.AMK_PATH_UNFUSED}


def _stream_ptr(stream: Optional[torch.cuda.Stream] = None) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


class KVCache:
    """KV cache [L][2][B][n_kv][max_seq][hd] bf16, owned by torch and borrowed by the library."""

    def __init__(self, model: "Model", batch: int, max_seq: int):
        cfg = model.cfg
        self.model = model
        self.batch, self.max_seq = batch, max_seq
        self.tensor = torch.zeros((cfg.n_layers, 2, batch, cfg.n_kv_heads, max_seq, cfg.head_dim),
                                  dtype=torch.bfloat16, device=model.device)
        lib = _lib.load()
        nbytes = C.c_size_t()
        _lib.check(lib.amk_kv_bytes(model.handle, batch, max_seq, C.byref(nbytes)), "amk_kv_bytes")
        assert nbytes.value == self.tensor.numel() * 2
        h = C.c_void_p()
        _lib.check(lib.amk_kv_alloc(model.handle, batch, max_seq, C.c_void_p(self.tensor.data_ptr()),
                                    nbytes.value, C.byref(h)), "amk_kv_alloc")
        self.handle = h

    def close(self):
        if self.handle:
            _lib.load().amk_kv_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Model:
    """A decoder model inside libamk. `weights` are host tensors from synth.make_weights (or
    any tensors of the documented shapes); they are uploaded, repacked by the library, and the
    uploaded copies released."""

    def __init__(self, cfg: Config, weights: Weights, path: str = "megakernel",
                 max_batch: Optional[int] = None, max_seq: Optional[int] = None,
                 schedule: Optional[bytes] = None, device: str = "cuda"):
        if not torch.cuda.is_available():
            raise RuntimeError("libamk needs a GPU: no HIP device is visible")
        self.cfg = cfg
        self.device = torch.device(device)
        self.lib = _lib.load()
        self.path = path
        self.max_batch = max_batch or cfg.batch
        self.max_seq = max_seq or cfg.max_seq
        self.c_cfg = _lib.make_config(cfg, self.max_batch, self.max_seq)
        dev = {}

        def up(t):
            if t is None:
                return None
            g = t.to(self.device, non_blocking=False).contiguous()
            dev[id(g)] = g
            return g

        layers = (_lib.amk_layer_weights * cfg.n_layers)()
        for l in range(cfg.n_layers):
            lw = layers[l]
            for m in MATS:
                setattr(lw, m, _ptr(up(weights.layers[l][m])))
            if cfg.wtype in ("int8", "int4"):
                for m in MATS:
                    setattr(lw, "s" + m[1], _ptr(up(weights.scales[l][m])))
            lw.attn_norm = _ptr(up(weights.attn_norm[l]))
            lw.mlp_norm = _ptr(up(weights.mlp_norm[l]))
        w = _lib.amk_weights()
        w.embed = _ptr(up(weights.embed))
        w.final_norm = _ptr(up(weights.final_norm))
        w.lm_head = _ptr(up(weights.lm_head))
        w.lm_head_scale = _ptr(up(weights.lm_head_scale))
        w.layers = layers
        h = C.c_void_p()
        blob = schedule if schedule is not None else None
        st = self.lib.amk_model_create(C.byref(self.c_cfg), C.byref(w), PATHS[path],
                                       blob, len(blob) if blob else 0, _stream_ptr(), C.byref(h))
        dev.clear()
        _lib.check(st, "amk_model_create")
        self.handle = h
        self.logits = None

    # ------------------------------------------------------------------------------------------
    def info(self) -> _lib.amk_model_info:
        out = _lib.amk_model_info()
        _lib.check(self.lib.amk_model_get_info(self.handle, C.byref(out)), "amk_model_get_info")
        return out

    def schedule(self) -> bytes:
        b = C.c_void_p()
        n = C.c_size_t()
        _lib.check(self.lib.amk_model_get_schedule(self.handle, C.byref(b), C.byref(n)),
                   "amk_model_get_schedule")
        try:
            return C.string_at(b, n.value)
        finally:
            self.lib.amk_blob_free(b)

    def set_schedule(self, blob: bytes) -> None:
        _lib.check(self.lib.amk_model_set_schedule(self.handle, blob, len(blob), _stream_ptr()),
                   "amk_model_set_schedule")

    def tune(self, kv: "KVCache", pos: int, rounds: int = 6, steps: int = 4,
             gain: float = 0.6) -> float:
        """Profile-guided re-tiling on the device (amk_model_tune); returns the mean step time
        (us) of the schedule it keeps installed."""
        best = C.c_double()
        _lib.check(self.lib.amk_model_tune(self.handle, kv.handle, pos, rounds, steps, float(gain),
                                           _stream_ptr(), C.byref(best)), "amk_model_tune")
        return best.value

    def enable_trace(self) -> torch.Tensor:
        """Turn on the megakernel's task trace; returns the device buffer it fills each step."""
        inf = self.info()
        buf = torch.zeros(4 * inf.n_tasks + inf.n_cu, dtype=torch.int64, device=self.device)
        _lib.check(self.lib.amk_trace_enable(self.handle, C.c_void_p(buf.data_ptr()),
                                             buf.numel() * 8), "amk_trace_enable")
        self._trace = buf
        return buf

    def kv(self, batch: Optional[int] = None, max_seq: Optional[int] = None) -> KVCache:
        return KVCache(self, batch or self.max_batch, max_seq or self.max_seq)

    def step(self, kv: KVCache, tokens: torch.Tensor, pos: int, logits: Optional[torch.Tensor] = None,
             next_out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """One decode step. tokens: device int32 [B]. Returns the device int32 next-token tensor."""
        B = tokens.numel()
        if next_out is None:
            next_out = torch.empty(B, dtype=torch.int32, device=self.device)
        st = self.lib.amk_decode_step(self.handle, kv.handle, C.c_void_p(tokens.data_ptr()), pos, B,
                                      C.c_void_p(_ptr(logits)) if logits is not None else None,
                                      C.c_void_p(next_out.data_ptr()), _stream_ptr())
        _lib.check(st, "amk_decode_step")
        return next_out

    def steps(self, kv: KVCache, tokens: torch.Tensor, pos, n_steps: int,
              logits: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """n_steps greedy decode steps in one launch (amk_decode_steps). tokens: device int32 [B];
        pos: one position for all sequences, or a sequence of B positions (amk_decode_steps_ragged).
        Returns the device int32 [n_steps, B] tokens; logits (if given): [n_steps, B, V] float32."""
        B = tokens.numel()
        if out is None:
            out = torch.empty((n_steps, B), dtype=torch.int32, device=self.device)
        if not isinstance(pos, int):
            pv = (C.c_int32 * B)(*[int(p) for p in pos])
            if len(pos) != B:
                raise ValueError("one position per sequence")
            st = self.lib.amk_decode_steps_ragged(
                self.handle, kv.handle, C.c_void_p(tokens.data_ptr()), pv, n_steps, B,
                C.c_void_p(_ptr(logits)) if logits is not None else None,
                C.c_void_p(out.data_ptr()), _stream_ptr())
            _lib.check(st, "amk_decode_steps_ragged")
            return out
        st = self.lib.amk_decode_steps(self.handle, kv.handle, C.c_void_p(tokens.data_ptr()), pos,
                                       n_steps, B,
                                       C.c_void_p(_ptr(logits)) if logits is not None else None,
                                       C.c_void_p(out.data_ptr()), _stream_ptr())
        _lib.check(st, "amk_decode_steps")
        return out

    def steps_noalloc(self, kv: KVCache, tokens: torch.Tensor, pos: int, n_steps: int,
                      logits: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """amk_decode_steps_noalloc: as steps() with one position, on the library's static
        per-GPU scratch array (the call allocates no device memory; `out` must then be given by
        callers that cannot allocate). Returns the device int32 [n_steps, B] tokens."""
        B = tokens.numel()
        if out is None:
            out = torch.empty((n_steps, B), dtype=torch.int32, device=self.device)
        st = self.lib.amk_decode_steps_noalloc(
            self.handle, kv.handle, C.c_void_p(tokens.data_ptr()), pos, n_steps, B,
            C.c_void_p(_ptr(logits)) if logits is not None else None, C.c_void_p(out.data_ptr()),
            _stream_ptr())
        _lib.check(st, "amk_decode_steps_noalloc")
        return out

    def prefill(self, kv: KVCache, tokens: torch.Tensor, pos0: int = 0, seq: int = 0,
                logits: Optional[torch.Tensor] = None, next_out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Process a prompt (device int32 [n]) of KV sequence `seq` at positions pos0 .. pos0 + n - 1
        (amk_prefill). Returns the device int32 [1] greedy next token; logits (if given): the last
        prompt token's float32 [V]."""
        if next_out is None:
            next_out = torch.empty(1, dtype=torch.int32, device=self.device)
        st = self.lib.amk_prefill(self.handle, kv.handle, seq, C.c_void_p(tokens.data_ptr()), pos0,
                                  tokens.numel(), C.c_void_p(_ptr(logits)) if logits is not None else None,
                                  C.c_void_p(next_out.data_ptr()), _stream_ptr())
        _lib.check(st, "amk_prefill")
        return next_out

    def sync(self):
        _lib.check(self.lib.amk_sync(self.handle, _stream_ptr()), "amk_sync")

    def close(self):
        if getattr(self, "handle", None):
            self.lib.amk_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
