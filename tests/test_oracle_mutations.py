"""Planted mistakes: each plausible error in the oracle's source must make at least one pin fail.

A mutant is built on the CPU by editing the oracle's source text and executing it as a fresh
module; the real oracle is never modified."""
import inspect
import types

import numpy as np
import pytest

from oracle import decoder as od
from persistent_decode_megakernel_amd import synth

import test_oracle_pins as pins

SRC = inspect.getsource(od)


def mutant(old: str, new: str) -> types.ModuleType:
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    m = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), m.__dict__)
    return m


def all_pins_pass(mod) -> bool:
    checks = [
        lambda: pins.pin_rmsnorm(mod),
        lambda: pins.pin_attention(mod),
        lambda: pins.pin_rope(mod),
        lambda: pins.pin_brute_force(synth.micro_config(L=2, d=64, nq=4, nkv=2, hd=16, F=80,
                                                        V=100), seed=1, mod=mod) < 1e-10,
        lambda: pins.pin_brute_force(synth.micro_config(L=1, d=64, nq=2, nkv=1, hd=32, F=96,
                                                        V=128), seed=2, with_prefill=True,
                                     mod=mod) < 1e-10,
        lambda: _argmax_pin(mod),
        lambda: _silu_pin(mod),
    ]
    for c in checks:
        try:
            if not c():
                return False
        except Exception:
            return False
    return True


def _argmax_pin(mod):
    lg = np.zeros((2, 10))
    lg[0, [2, 7]] = 1.0
    lg[1, 9] = 3.0
    return list(mod.argmax_lowest(lg)) == [2, 9]


def _silu_pin(mod):
    return abs(mod.silu(np.array([1.0]))[0] - 1 / (1 + np.exp(-1.0))) < 1e-15


def test_unmutated_oracle_passes_all_pins():
    assert all_pins_pass(od)


MUTATIONS = {
    "eps outside sqrt": ("gain * (r / np.sqrt(ms + eps))", "gain * (r / (np.sqrt(ms) + eps))"),
    "sum instead of mean": ("ms = np.mean(r * r, axis=-1, keepdims=True)",
                            "ms = np.sum(r * r, axis=-1, keepdims=True)"),
    "gain dropped": ("return gain * (r / np.sqrt(ms + eps))", "return r / np.sqrt(ms + eps)"),
    "rope interleaved pairs": ("a, b = u[..., :half], u[..., half:]",
                               "a, b = u[..., 0::2], u[..., 1::2]"),
    "rope sign": ("[a * c - b * s, b * c + a * s]", "[a * c + b * s, b * c - a * s]"),
    "rope frequency base": ("omega = theta ** (-2.0 * j / head_dim)",
                            "omega = theta ** (-1.0 * j / head_dim)"),
    "no attention scale": ("s = (K @ q) / math.sqrt(q.shape[-1])", "s = K @ q"),
    "softmax without normalisation": ("return e / np.sum(e, axis=-1, keepdims=True)",
                                      "return e"),
    "silu as sigmoid": ("return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    "gqa grouping modulo": ("for h in range(g * group, (g + 1) * group):",
                            "for h in range(g, nq, nkv):"),
    "no causal current token": ("K = bf16_to_float(kv[l, 0, b, g, : pos + 1, :], dt)",
                                "K = bf16_to_float(kv[l, 0, b, g, : max(pos, 1), :], dt)"),
    "k not rotated": ("k = apply_rope(k, pos, theta)", "k = k"),
    "attention residual dropped": (
        "r = r + self.matvec((l, \"wo\"), lw[\"wo\"], lw.get(\"so\"), o.reshape(B, nq * hd))",
        "r = self.matvec((l, \"wo\"), lw[\"wo\"], lw.get(\"so\"), o.reshape(B, nq * hd))"),
    "gate and up swapped": ("r = r + self.matvec((l, \"wd\"), lw[\"wd\"], lw.get(\"sd\"), silu(gate) * up)",
                            "r = r + self.matvec((l, \"wd\"), lw[\"wd\"], lw.get(\"sd\"), silu(up) * gate)"),
    "mlp norm uses attn gain": ("x = rmsnorm(r, self._vec(lw[\"mlp_norm\"]), eps)",
                                "x = rmsnorm(r, self._vec(lw[\"attn_norm\"]), eps)"),
    "final norm skipped": ("x = rmsnorm(r, self._vec(w[\"final_norm\"]), eps)", "x = r"),
    "square weight transposed": ("y = x @ m.T", "y = x @ (m if m.shape[0] == m.shape[1] else m.T)"),
    "int8 scale dropped": ("y = y * sc", "y = y"),
    "int4 nibbles swapped": ("out[:, 0::2] = lo\n    out[:, 1::2] = hi", "out[:, 0::2] = hi\n    out[:, 1::2] = lo"),
    "int4 not sign extended": ("lo = np.where(lo >= 8, lo - 16, lo).astype(np.int8)", "lo = lo"),
    "int4 groups interleaved": ("return q * np.repeat(sc, group, axis=1)",
                                "return q * np.tile(sc, (1, group))"),
    "int4 group too wide": ("return q * np.repeat(sc, group, axis=1)",
                            "return q * np.repeat(np.repeat(sc[:, ::2], 2, axis=1), group, axis=1)"),
    "argmax highest tie": ("return np.argmax(logits, axis=-1).astype(np.int32)",
                           "return (logits.shape[-1] - 1 - np.argmax(logits[..., ::-1], axis=-1)).astype(np.int32)"),
    "bf16 truncation": ("rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)",
                        "rounded = u >> np.uint64(16)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    if name == "int8 scale dropped":
        m = mutant(old, new)
        cfg = synth.micro_config(L=1, d=64, nq=2, nkv=1, hd=32, F=96, V=128, wtype="int8")
        w = synth.make_weights(cfg, 5)
        params, wn = synth.oracle_inputs(w)
        kv = np.zeros((1, 2, 1, 1, 3, 32), np.uint16)
        a = pins._incremental(params, wn, [1, 2, 3], kv, 0, mod=m)
        b = pins.brute_force_logits(params, wn, [1, 2, 3])
        assert np.max(np.abs(a - b)) > 1e-6
        return
    if name.startswith("int4"):
        m = mutant(old, new)
        ok = True
        try:
            ok = pins.pin_int4(m) and pins.pin_int4_brute_force(m) < 1e-12
        except Exception:
            ok = False
        assert not ok
        return
    if name == "bf16 truncation":
        m = mutant(old, new)
        x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
        import torch
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert not np.array_equal(m.float_to_bf16(x), ref)
        return
    assert not all_pins_pass(mutant(old, new))
