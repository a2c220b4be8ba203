"""Plain CPU reference for one autoregressive decode step of a Llama-style decoder.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this module:
only the tests, the package's smoke check and the bench's CPU-baseline leg use it. It shares no
code with the HIP path; it reads the same seeded input bytes.

What is computed, and where it comes from:
  * the pages (Ada-MK technical summary, "Methodology", Phase I) name the graph that the
    megakernel covers as the Transformer decoder plus the LM head, and the AutoMegaKernel
    abstract (page 5 of the set) names HuggingFace Llama-family models under greedy decoding;
  * the operators themselves are the textbook Llama decoder: RMSNorm (Zhang & Sennrich, 2019),
    rotary position embedding with half-split pairs (Su et al., 2021; the HF Llama convention),
    grouped-query attention (Ainslie et al., 2023), SwiGLU MLP (Shazeer, 2020), no biases,
    greedy argmax with ties broken towards the lowest index.

Precision: computed in float64 by default (float32 on request). Weights are read exactly from
their bfloat16 / int8 / packed int4 bit patterns.

W4A16 (the Ada-MK technical summary, "Key Contributions" item 4 and "Experimental Results", names
GPTQ-W4A16 and nothing of its format): read here as symmetric 4-bit integers q in [-8, 7] with
one float32 scale per output row and group of G consecutive inputs, W[o, i] = s[o, i // G] *
q[o, i]; activations stay floating point. Storage: uint8 [out, in / 2], element 2j in the low
nibble of byte j and 2j + 1 in the high nibble, each nibble two's complement. The only rounding the method itself fixes is the bf16 KV
cache: newly appended K/V rows are rounded to bf16 (round-to-nearest-even) before they are
stored, exactly as a bf16 cache holds them. RoPE angles are always formed in float64.

Data layout of the KV cache (shared with the library as an input/output convention, not code):
    kv[l][0 = K, 1 = V][b][kv_head][position][head_dim], bfloat16 bit patterns (uint16).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


# --------------------------------------------------------------------------------------------
# bfloat16 bit patterns
# --------------------------------------------------------------------------------------------
def bf16_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: the 16 bits are the top half of an IEEE float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(dtype)


def float_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16, ties to even, returning bit patterns (uint16).

    Reading taken: the pages fix only that the KV cache is bf16 (they decode HuggingFace
    Llama-family models in bf16, the AutoMegaKernel abstract). A value stored there is a matrix
    product's result, which such a model accumulates in float32 before storing it in bf16. So the
    value is first rounded to float32, then to bf16 with round-to-nearest-even (the rounding of
    torch's and numpy's bf16 casts): add 0x7FFF plus the lowest kept bit and drop the low 16 bits.
    NaN inputs are not expected and not handled.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


# --------------------------------------------------------------------------------------------
# operators
# --------------------------------------------------------------------------------------------
def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 [out, in / 2] -> int8 [out, in]: byte j holds elements 2j (low nibble) and 2j + 1
    (high nibble), each a 4-bit two's complement integer."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo).astype(np.int8)
    hi = np.where(hi >= 8, hi - 16, hi).astype(np.int8)
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequant_int4(packed: np.ndarray, scales: np.ndarray, group: int, dtype=np.float64) -> np.ndarray:
    """W[o, i] = scales[o, i // group] * q[o, i] (exact in float64: a 4-bit integer times a
    float32)."""
    q = unpack_int4(packed).astype(dtype)
    sc = np.asarray(scales, dtype=np.float32).astype(dtype)
    assert sc.shape == (q.shape[0], q.shape[1] // group)
    return q * np.repeat(sc, group, axis=1)


def rmsnorm(r: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """y_i = g_i * r_i / sqrt(mean_j(r_j^2) + eps); the mean runs over the last axis."""
    ms = np.mean(r * r, axis=-1, keepdims=True)
    return gain * (r / np.sqrt(ms + eps))


def rope_cos_sin(pos: int, head_dim: int, theta: float):
    """cos/sin of the rotation angles pos * theta^(-2j/head_dim), j < head_dim/2, in float64."""
    half = head_dim // 2
    j = np.arange(half, dtype=np.float64)
    omega = theta ** (-2.0 * j / head_dim)
    phi = float(pos) * omega
    return np.cos(phi), np.sin(phi)


def apply_rope(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate each head vector (last axis) by position `pos`; dimension j pairs with j + hd/2."""
    hd = u.shape[-1]
    half = hd // 2
    c, s = rope_cos_sin(pos, hd, theta)
    c = c.astype(u.dtype)
    s = s.astype(u.dtype)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum exp(s - max s) over the last axis."""
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """One query vector against ctx keys/values: softmax(K q / sqrt(hd)) V."""
    s = (K @ q) / math.sqrt(q.shape[-1])
    return softmax(s) @ V


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Index of the largest logit per row; among equal maxima the lowest index wins."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """top-1 minus top-2 logit per row (0 when the maximum is attained twice)."""
    part = np.sort(logits, axis=-1)
    return part[..., -1] - part[..., -2]


# --------------------------------------------------------------------------------------------
# model
# --------------------------------------------------------------------------------------------
class Decoder:
    """A Llama-style decoder given as raw weight bytes.

    params: dict with n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, rms_eps,
            rope_theta, int8 (bool), int4 (bool), group (int4 inputs per scale group).
    weights: dict with
        embed [V, d] bf16 bits; final_norm [d] bf16 bits;
        lm_head [V, d] (bf16 bits, int8, or packed int4 [V, d / 2]) or None when tied to the
        embedding; lm_head_scale [V] float32 (int8) or [V, d / group] (int4);
        layers: list of dicts wq wk wv wo wg wu wd ([out, in]; bf16 bits or int8; int4: packed
                uint8 [out, in / 2]), sq sk sv so sg su sd (float32 [out] for int8,
                [out, in / group] for int4), attn_norm, mlp_norm (bf16 bits).
    """

    def __init__(self, params: Dict, weights: Dict, dtype=np.float64,
                 cache_bytes: int = 8 << 30):
        self.p = dict(params)
        self.w = weights
        self.dtype = dtype
        self._cache: Dict = {}
        self._cache_left = cache_bytes

    # weights in the compute dtype -----------------------------------------------------------
    def _mat(self, key, bits: np.ndarray, scale: Optional[np.ndarray]):
        """Return (matrix, scale) in the compute dtype; int8 values convert exactly; int4 matrices
        are dequantised with their group scales (the returned scale is then None)."""
        if key in self._cache:
            return self._cache[key]
        if bits.dtype == np.uint8:
            m = dequant_int4(bits, scale, int(self.p["group"]), self.dtype)
            sc = None
        elif bits.dtype == np.int8:
            m = bits.astype(self.dtype)
            sc = np.asarray(scale, dtype=np.float32).astype(self.dtype)
        else:
            m = bf16_to_float(bits, self.dtype)
            sc = None
        nbytes = m.nbytes
        if nbytes <= self._cache_left:
            self._cache[key] = (m, sc)
            self._cache_left -= nbytes
        return m, sc

    def _vec(self, bits):
        return bf16_to_float(bits, self.dtype)

    def matvec(self, key, bits, scale, x):
        """y = W x for a batch of row vectors x [B, in]; int8: y_o = s_o * sum_i Q_oi x_i."""
        m, sc = self._mat(key, bits, scale)
        y = x @ m.T
        if sc is not None:
            y = y * sc
        return y

    # one step --------------------------------------------------------------------------------
    def step(self, kv: np.ndarray, tokens: np.ndarray, pos: int) -> np.ndarray:
        """Decode one token per sequence at position `pos`.

        kv: uint16 [L][2][B][n_kv][max_seq][hd], updated in place (slot `pos` is written).
        tokens: int [B]. Returns logits [B, V] in the compute dtype.
        """
        p, w, dt = self.p, self.w, self.dtype
        L, d = p["n_layers"], p["hidden"]
        nq, nkv, hd = p["n_heads"], p["n_kv_heads"], p["head_dim"]
        eps, theta = p["rms_eps"], p["rope_theta"]
        group = nq // nkv
        tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
        B = tokens.shape[0]
        assert kv.shape[2] == B and pos < kv.shape[4]

        r = self._vec(w["embed"][tokens])  # [B, d]
        for l in range(L):
            lw = w["layers"][l]
            x = rmsnorm(r, self._vec(lw["attn_norm"]), eps)
            q = self.matvec((l, "wq"), lw["wq"], lw.get("sq"), x).reshape(B, nq, hd)
            k = self.matvec((l, "wk"), lw["wk"], lw.get("sk"), x).reshape(B, nkv, hd)
            v = self.matvec((l, "wv"), lw["wv"], lw.get("sv"), x).reshape(B, nkv, hd)
            q = apply_rope(q, pos, theta)
            k = apply_rope(k, pos, theta)
            kv[l, 0, :, :, pos, :] = float_to_bf16(k)
            kv[l, 1, :, :, pos, :] = float_to_bf16(v)
            o = np.empty((B, nq, hd), dtype=dt)
            for b in range(B):
                for g in range(nkv):
                    K = bf16_to_float(kv[l, 0, b, g, : pos + 1, :], dt)
                    V = bf16_to_float(kv[l, 1, b, g, : pos + 1, :], dt)
                    for h in range(g * group, (g + 1) * group):
                        o[b, h] = attend(q[b, h], K, V)
            r = r + self.matvec((l, "wo"), lw["wo"], lw.get("so"), o.reshape(B, nq * hd))
            x = rmsnorm(r, self._vec(lw["mlp_norm"]), eps)
            gate = self.matvec((l, "wg"), lw["wg"], lw.get("sg"), x)
            up = self.matvec((l, "wu"), lw["wu"], lw.get("su"), x)
            r = r + self.matvec((l, "wd"), lw["wd"], lw.get("sd"), silu(gate) * up)
        x = rmsnorm(r, self._vec(w["final_norm"]), eps)
        lm = w["lm_head"] if w.get("lm_head") is not None else w["embed"]
        return self.matvec(("lm",), lm, w.get("lm_head_scale"), x)
