"""Pins for the CPU oracle: each check ties an oracle function to something other than itself
(closed forms, invariants, library routines, brute force on tiny inputs).

Every test here runs on the CPU (not marked gpu)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import decoder as od
from persistent_decode_megakernel_amd import synth

EPS = 1e-5


# ---------------------------------------------------------------------------------------------
# P1 RMSNorm: constant vector closed form, eps inside the sqrt, gain after normalisation
# ---------------------------------------------------------------------------------------------
def pin_rmsnorm(mod=od):
    d = 64
    g = np.ones(d)
    # r = c*1 => y = c / sqrt(c^2 + eps)
    for c, want in [(1.0, 0.99999500003750), (1e-3, 0.30151134457776), (0.0, 0.0),
                    (-2.0, -0.99999875000234)]:
        y = mod.rmsnorm(np.full((1, d), c), g, EPS)
        if not np.allclose(y, want, rtol=1e-12, atol=1e-14):
            return False
    # gain multiplies after normalisation; scale invariance of the normalised part
    rng = np.random.default_rng(1)
    r = rng.standard_normal((3, d))
    gain = rng.standard_normal(d)
    y = mod.rmsnorm(r, gain, 0.0)
    if not np.allclose(np.sqrt(np.mean((y / gain) ** 2, axis=-1)), 1.0, rtol=1e-12):
        return False
    # second opinion: torch's rms_norm
    t = F.rms_norm(torch.from_numpy(r), (d,), torch.from_numpy(gain), eps=EPS).numpy()
    return np.allclose(mod.rmsnorm(r, gain, EPS), t, rtol=1e-12, atol=1e-13)


def test_p1_rmsnorm():
    assert pin_rmsnorm()


# ---------------------------------------------------------------------------------------------
# P2 softmax
# ---------------------------------------------------------------------------------------------
def test_p2_softmax():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((5, 37)) * 10
    a = oracle.softmax(s)
    assert np.allclose(a.sum(-1), 1.0, atol=1e-14)
    assert np.allclose(oracle.softmax(s + 123.25), a, atol=1e-14)
    s1 = np.zeros(9)
    s1[4] = 100.0
    assert np.allclose(oracle.softmax(s1), np.eye(9)[4], atol=1e-40)
    # float32 rows sum to 1 within 1e-6
    a32 = oracle.softmax(s.astype(np.float32))
    assert np.all(np.abs(a32.sum(-1) - 1) < 1e-6)


# ---------------------------------------------------------------------------------------------
# P3 attention: single key returns V exactly; equal keys give the mean of V; torch SDPA
# ---------------------------------------------------------------------------------------------
def pin_attention(mod=od):
    rng = np.random.default_rng(3)
    hd = 64
    q = rng.standard_normal(hd)
    K = rng.standard_normal((1, hd))
    V = rng.standard_normal((1, hd))
    if not np.array_equal(mod.attend(q, K, V), V[0]):
        return False
    K = np.repeat(rng.standard_normal((1, hd)), 7, axis=0)
    V = rng.standard_normal((7, hd))
    if not np.allclose(mod.attend(q, K, V), V.mean(0), atol=1e-14):
        return False
    # second opinion: torch SDPA (scale 1/sqrt(hd)) on random data
    K = rng.standard_normal((13, hd))
    V = rng.standard_normal((13, hd))
    t = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None],
                                       torch.from_numpy(K)[None, None],
                                       torch.from_numpy(V)[None, None])[0, 0, 0].numpy()
    return np.allclose(mod.attend(q, K, V), t, atol=1e-12)


def test_p3_attention():
    assert pin_attention()


# ---------------------------------------------------------------------------------------------
# P4 RoPE
# ---------------------------------------------------------------------------------------------
def pin_rope(mod=od):
    rng = np.random.default_rng(4)
    for hd in (64, 128):
        u = rng.standard_normal((3, hd))
        for p in (0, 1, 7, 2047, 4159):
            ru = mod.apply_rope(u, p, 10000.0)
            if not np.allclose(np.linalg.norm(ru, axis=-1), np.linalg.norm(u, axis=-1),
                               rtol=1e-12):
                return False
        if not np.array_equal(mod.apply_rope(u, 0, 10000.0), u):  # R_0 = I exactly
            return False
        # e_0 -> cos(p) e_0 + sin(p) e_{hd/2}: omega_0 = 1, pairs are (j, j + hd/2)
        e0 = np.zeros(hd)
        e0[0] = 1.0
        for p in (1, 5, 100):
            want = np.zeros(hd)
            want[0], want[hd // 2] = math.cos(p), math.sin(p)
            if not np.allclose(mod.apply_rope(e0, p, 10000.0), want, atol=1e-15):
                return False
        # relative-position property <R_m q, R_n k> depends on m - n only
        q, k = rng.standard_normal(hd), rng.standard_normal(hd)
        a = mod.apply_rope(q, 10, 1e4) @ mod.apply_rope(k, 3, 1e4)
        b = mod.apply_rope(q, 1007, 1e4) @ mod.apply_rope(k, 1000, 1e4)
        if not abs(a - b) < 1e-9:
            return False
    # frequencies: omega_1 and omega_{hd/2-1}; cos(p*omega_j) at p = 1 gives omega via acos
    for hd, w1, wl in ((64, 0.74989420933246, 1.3335214321633e-4),
                       (128, 0.86596432336007, 1.1547819846894e-4)):
        c, s = mod.rope_cos_sin(1, hd, 10000.0)
        if not (abs(math.atan2(s[1], c[1]) - w1) < 1e-12
                and abs(math.atan2(s[-1], c[-1]) - wl) < 1e-15):
            return False
    return True


def test_p4_rope():
    assert pin_rope()


# ---------------------------------------------------------------------------------------------
# SiLU and bf16 conversions
# ---------------------------------------------------------------------------------------------
def test_silu():
    z = np.array([0.0, 1.0, -1.0, 20.0, -20.0])
    want = np.array([0.0, 1 / (1 + math.exp(-1)), -1 / (1 + math.e), 20 / (1 + math.exp(-20)),
                     -20 / (1 + math.exp(20))])
    assert np.allclose(oracle.silu(z), want, rtol=1e-15, atol=0)
    zz = np.random.default_rng(5).standard_normal(100) * 4
    assert np.allclose(oracle.silu(zz), F.silu(torch.from_numpy(zz)).numpy(), rtol=1e-14)


def test_bf16_roundtrip_and_rne():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    mine = oracle.float_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert np.array_equal(oracle.bf16_to_float(oracle.float_to_bf16(ties)),
                          np.array([1.0, 1 + 2 ** -6, -1.0]))
    bits = rng.integers(0, 2 ** 16, 1000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite values
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_to_float(bits, np.float32), vals)


# ---------------------------------------------------------------------------------------------
# P10 argmax
# ---------------------------------------------------------------------------------------------
def test_p10_argmax():
    lg = np.zeros((3, 50))
    lg[0, 17] = 5.0
    lg[1, [3, 9, 40]] = 2.0
    lg[2] = -1.0
    assert list(oracle.argmax_lowest(lg)) == [17, 3, 0]
    assert np.allclose(oracle.top2_margin(lg), [5.0, 0.0, 0.0])


# ---------------------------------------------------------------------------------------------
# brute-force full recompute (P5) written independently: whole sequences, causal masks, RoPE by
# complex multiplication, bf16 rounding of K/V through torch.
# ---------------------------------------------------------------------------------------------
def _bf16_round(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _nibbles(packed):
    """Signed 4-bit values of a packed [out, in / 2] byte array, element by element: byte j of a
    row holds element 2j in its low and 2j + 1 in its high nibble."""
    rows, half = packed.shape
    out = np.zeros((rows, 2 * half), dtype=np.int64)
    for o in range(rows):
        for j in range(half):
            b = int(packed[o, j])
            for k, nib in enumerate((b & 15, b >> 4)):
                out[o, 2 * j + k] = nib - 16 if nib >= 8 else nib
    return out


def _int4_dense(packed, scales, group):
    """Dense float64 matrix of an int4 weight, one scale group (a column block) at a time."""
    q = _nibbles(packed).astype(np.float64)
    for g in range(q.shape[1] // group):
        q[:, g * group:(g + 1) * group] *= np.asarray(scales, np.float64)[:, g:g + 1]
    return q


def brute_force_logits(params, w, tokens, prefill_k=None, prefill_v=None):
    """Logits at every fed position, recomputing the whole prefix (no cache).
    prefill_k/v: [L][n_kv][P][hd] values taken as already-rotated keys and plain values."""
    L, d = params["n_layers"], params["hidden"]
    nq, nkv, hd = params["n_heads"], params["n_kv_heads"], params["head_dim"]
    theta, eps = params["rope_theta"], params["rms_eps"]
    P = 0 if prefill_k is None else prefill_k.shape[2]
    T = len(tokens)
    pos = np.arange(P, P + T)

    def f(bits):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
            np.float64)

    def mat(lw, m):
        W = lw[m]
        if W.dtype == np.uint8:
            return _int4_dense(W, lw["s" + m[1]], params["group"])
        if W.dtype == np.int8:
            return W.astype(np.float64) * lw["s" + m[1]].astype(np.float64)[:, None]
        return f(W)

    def norm(X, g):
        return X / np.sqrt((X ** 2).mean(-1, keepdims=True) + eps) * f(g)

    def rot(X):  # X [T, heads, hd]
        half = hd // 2
        ang = pos[:, None] * theta ** (-np.arange(half) * 2.0 / hd)[None, :]
        z = (X[..., :half] + 1j * X[..., half:]) * np.exp(1j * ang)[:, None, :]
        return np.concatenate([z.real, z.imag], -1)

    R = f(w["embed"])[np.asarray(tokens)]
    for l in range(L):
        lw = w["layers"][l]
        X = norm(R, lw["attn_norm"])
        Q = rot((X @ mat(lw, "wq").T).reshape(T, nq, hd))
        Kn = _bf16_round(rot((X @ mat(lw, "wk").T).reshape(T, nkv, hd)))
        Vn = _bf16_round((X @ mat(lw, "wv").T).reshape(T, nkv, hd))
        if P:
            Kall = np.concatenate([prefill_k[l].transpose(1, 0, 2), Kn], 0)
            Vall = np.concatenate([prefill_v[l].transpose(1, 0, 2), Vn], 0)
        else:
            Kall, Vall = Kn, Vn
        O = np.zeros((T, nq, hd))
        mask = np.arange(P + T)[None, :] <= pos[:, None]  # [T, P+T]
        for h in range(nq):
            g = h // (nq // nkv)
            S = Q[:, h] @ Kall[:, g].T / math.sqrt(hd)
            S = np.where(mask, S, -np.inf)
            A = np.exp(S - S.max(-1, keepdims=True))
            A /= A.sum(-1, keepdims=True)
            O[:, h] = A @ Vall[:, g]
        R = R + O.reshape(T, nq * hd) @ mat(lw, "wo").T
        X = norm(R, lw["mlp_norm"])
        G, U = X @ mat(lw, "wg").T, X @ mat(lw, "wu").T
        R = R + (G / (1 + np.exp(-G)) * U) @ mat(lw, "wd").T
    X = norm(R, w["final_norm"])
    if w.get("lm_head") is None:
        lm = f(w["embed"])
    elif w["lm_head"].dtype == np.uint8:
        lm = _int4_dense(w["lm_head"], w["lm_head_scale"], params["group"])
    elif w["lm_head"].dtype == np.int8:
        lm = w["lm_head"].astype(np.float64) * w["lm_head_scale"].astype(np.float64)[:, None]
    else:
        lm = f(w["lm_head"])
    return X @ lm.T


def _incremental(params, w, tokens, kv, pos0, dtype=np.float64, mod=od):
    dec = mod.Decoder(params, w, dtype=dtype)
    out = []
    for i, t in enumerate(tokens):
        out.append(dec.step(kv, np.array([t]), pos0 + i)[0])
    return np.stack(out)


MICROS = [
    dict(L=1, d=8, nq=1, nkv=1, hd=8, F=16, V=32),
    dict(L=1, d=64, nq=2, nkv=1, hd=32, F=96, V=128),
    dict(L=2, d=64, nq=4, nkv=2, hd=16, F=80, V=100),
]


def pin_brute_force(cfg, seed=0, n_tok=6, with_prefill=False, mod=od):
    w = synth.make_weights(cfg, seed, random_gains=True)
    params, wn = synth.oracle_inputs(w)
    rng = np.random.default_rng(seed)
    tokens = rng.integers(0, cfg.vocab, n_tok)
    P = 5 if with_prefill else 0
    kv = np.zeros((cfg.n_layers, 2, 1, cfg.n_kv_heads, P + n_tok, cfg.head_dim), np.uint16)
    pk = pv = None
    if P:
        kvp = synth.make_kv(cfg.replace(prefill=P), P + n_tok, seed)
        kv[:] = synth.bf16_to_numpy_bits(kvp)
        pk = oracle.bf16_to_float(kv[:, 0, 0, :, :P, :])
        pv = oracle.bf16_to_float(kv[:, 1, 0, :, :P, :])
    got = _incremental(params, wn, tokens, kv, P, mod=mod)
    want = brute_force_logits(params, wn, tokens, pk, pv)
    return float(np.max(np.abs(got - want)))


@pytest.mark.parametrize("m", MICROS)
@pytest.mark.parametrize("with_prefill", [False, True])
def test_p5_brute_force_micro(m, with_prefill):
    cfg = synth.micro_config(**m)
    assert pin_brute_force(cfg, seed=1, with_prefill=with_prefill) < 1e-10


def test_p5_brute_force_tiny_config():
    cfg = synth.get_config("tiny")
    assert pin_brute_force(cfg, seed=0, n_tok=5) < 1e-9


# ---------------------------------------------------------------------------------------------
# P6 zero layers: logits = W_lm rmsnorm(E[tok], g_f)
# ---------------------------------------------------------------------------------------------
def test_p6_zero_layers_closed_form():
    cfg = synth.micro_config(L=2, d=64, nq=2, nkv=1, hd=32, F=96, V=128)
    w = synth.make_weights(cfg, 3, random_gains=True)
    params, wn = synth.oracle_inputs(w)
    for lw in wn["layers"]:
        for m in synth.MATS:
            lw[m] = np.zeros_like(lw[m])
    kv = np.zeros((2, 2, 1, 1, 4, 32), np.uint16)
    lg = oracle.Decoder(params, wn).step(kv, np.array([7]), 2)[0]
    e = oracle.bf16_to_float(wn["embed"][7])
    g = oracle.bf16_to_float(wn["final_norm"])
    want = oracle.bf16_to_float(wn["lm_head"]) @ (g * e / math.sqrt(np.mean(e * e) + EPS))
    assert np.allclose(lg, want, rtol=1e-12, atol=1e-14)
    # zero V projection -> attention contributes zero -> appended V rows are exactly zero
    assert np.all(kv[:, 1, :, :, 2, :] == 0)


# ---------------------------------------------------------------------------------------------
# P7 GQA == MHA with K/V rows repeated per group
# ---------------------------------------------------------------------------------------------
def test_p7_gqa_equals_repeated_mha():
    cfg = synth.micro_config(L=2, d=64, nq=4, nkv=2, hd=16, F=80, V=100)
    w = synth.make_weights(cfg, 4)
    params, wn = synth.oracle_inputs(w)
    params_mha = dict(params, n_kv_heads=4)
    wm = {**wn, "layers": []}
    for lw in wn["layers"]:
        d = dict(lw)
        for m in ("wk", "wv"):
            heads = lw[m].reshape(2, 16, 64)
            d[m] = np.repeat(heads, 2, axis=0).reshape(64, 64)
        wm["layers"].append(d)
    toks = [5, 17, 99, 3]
    kv1 = np.zeros((2, 2, 1, 2, 4, 16), np.uint16)
    kv2 = np.zeros((2, 2, 1, 4, 4, 16), np.uint16)
    a = _incremental(params, wn, toks, kv1, 0)
    b = _incremental(params_mha, wm, toks, kv2, 0)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# P8 int8 path == bf16-valued path with dequantised weights (float64, identity)
# P9 tied head == untied head holding a copy of the embedding
# ---------------------------------------------------------------------------------------------
def test_p8_int8_equals_dequantised():
    cfg = synth.micro_config(L=2, d=64, nq=2, nkv=1, hd=32, F=96, V=128, wtype="int8")
    w = synth.make_weights(cfg, 5)
    params, wn = synth.oracle_inputs(w)
    toks = [1, 2, 3]
    kv = np.zeros((2, 2, 1, 1, 3, 32), np.uint16)
    a = _incremental(params, wn, toks, kv, 0)
    b = brute_force_logits(params, wn, toks)  # dequantises as s_o * Q_oi up front
    assert np.max(np.abs(a - b)) < 1e-12


# ---------------------------------------------------------------------------------------------
# P12 W4A16: unpacking and group scales by a hand-computed example, the decoder against the brute
# force (its own per-group dequantisation), and W4A16 with one scale per row == W8A16
# ---------------------------------------------------------------------------------------------
def pin_int4(mod=od):
    # row 0: q = [1, -1, 2, 3] -> bytes 0xF1 (1, -1), 0x32 (2, 3); row 1: q = [-8, 7, 0, -2] ->
    # bytes 0x78 (-8, 7), 0xE0 (0, -2); groups of 2 inputs: scales [[0.5, 2], [4, 0.25]]
    packed = np.array([[0xF1, 0x32], [0x78, 0xE0]], dtype=np.uint8)
    if list(mod.unpack_int4(packed).ravel()) != [1, -1, 2, 3, -8, 7, 0, -2]:
        return False
    W = mod.dequant_int4(packed, np.array([[0.5, 2.0], [4.0, 0.25]], np.float32), 2)
    return np.array_equal(W, np.array([[0.5, -0.5, 4.0, 6.0], [-32.0, 28.0, 0.0, -0.5]]))


def test_p12_int4_known_answer():
    assert pin_int4()
    # every byte value: the low nibble is element 2j, the high nibble element 2j + 1
    allb = np.arange(256, dtype=np.uint8)[None, :]
    q = od.unpack_int4(allb)
    assert np.array_equal(q, _nibbles(allb))
    assert q.min() == -8 and q.max() == 7


def pin_int4_brute_force(mod=od, seed=8):
    cfg = synth.micro_config(L=2, d=64, nq=4, nkv=2, hd=16, F=96, V=100, wtype="int4", group=32)
    w = synth.make_weights(cfg, seed)
    params, wn = synth.oracle_inputs(w)
    toks = [5, 17, 99, 0]
    kv = np.zeros((2, 2, 1, 2, len(toks), 16), np.uint16)
    a = _incremental(params, wn, toks, kv, 0, mod=mod)
    b = brute_force_logits(params, wn, toks)
    return float(np.max(np.abs(a - b)))


def test_p12_int4_decoder_equals_brute_force():
    assert pin_int4_brute_force() < 1e-12


def test_p12_int4_with_row_scales_equals_int8():
    """Every group of a row given the same scale: W4A16 reduces to W8A16 with the same integers
    and that per-row scale (the int8 path is pinned against the brute force by P8)."""
    cfg4 = synth.micro_config(L=2, d=64, nq=2, nkv=1, hd=32, F=96, V=128, wtype="int4", group=16)
    w = synth.make_weights(cfg4, 9)
    params4, wn4 = synth.oracle_inputs(w)
    params8 = dict(params4, int4=False, int8=True, group=0)

    def to_row_scales(packed, sc):
        row = np.asarray(sc, np.float32)[:, :1]
        return np.repeat(row, sc.shape[1], axis=1), _nibbles(packed).astype(np.int8), row[:, 0].copy()

    layers4, layers8 = [], []
    for lw in wn4["layers"]:
        l4, l8 = dict(lw), dict(lw)
        for m in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            s4, q8, s8 = to_row_scales(lw[m], lw["s" + m[1]])
            l4["s" + m[1]] = s4
            l8[m], l8["s" + m[1]] = q8, s8
        layers4.append(l4)
        layers8.append(l8)
    s4, q8, s8 = to_row_scales(wn4["lm_head"], wn4["lm_head_scale"])
    wa = dict(wn4, layers=layers4, lm_head_scale=s4)
    wb = dict(wn4, layers=layers8, lm_head=q8, lm_head_scale=s8)
    toks = [3, 70, 12]
    kv1 = np.zeros((2, 2, 1, 1, 3, 32), np.uint16)
    kv2 = kv1.copy()
    a = _incremental(params4, wa, toks, kv1, 0)
    b = _incremental(params8, wb, toks, kv2, 0)
    assert np.max(np.abs(a - b)) < 1e-12


def test_p9_tied_equals_copy():
    cfg = synth.micro_config(L=1, d=64, nq=2, nkv=1, hd=32, F=96, V=128, tied=True)
    w = synth.make_weights(cfg, 6)
    params, wn = synth.oracle_inputs(w)
    assert wn["lm_head"] is None
    wc = dict(wn, lm_head=wn["embed"].copy())
    kv1 = np.zeros((1, 2, 1, 1, 3, 32), np.uint16)
    kv2 = kv1.copy()
    assert np.array_equal(_incremental(params, wn, [4, 5], kv1, 0),
                          _incremental(params, wc, [4, 5], kv2, 0))


# ---------------------------------------------------------------------------------------------
# P11 determinism and batch independence
# ---------------------------------------------------------------------------------------------
def test_p11_batch_rows_are_independent():
    cfg = synth.micro_config(L=2, d=64, nq=4, nkv=2, hd=16, F=80, V=100, batch=3, prefill=4)
    w = synth.make_weights(cfg, 7)
    params, wn = synth.oracle_inputs(w)
    kv = synth.bf16_to_numpy_bits(synth.make_kv(cfg, 8, 7)).copy()
    toks = np.array([3, 50, 99])
    lg = oracle.Decoder(params, wn).step(kv.copy(), toks, 4)
    for b in range(3):
        kb = kv[:, :, b:b + 1].copy()
        lb = oracle.Decoder(params, wn).step(kb, toks[b:b + 1], 4)
        assert np.max(np.abs(lb[0] - lg[b])) < 1e-13  # BLAS gemm vs gemv rounding only
    w2 = synth.make_weights(cfg, 7)
    assert torch.equal(w2.layers[1]["wd"], w.layers[1]["wd"])


# ---------------------------------------------------------------------------------------------
# independent torch forward (second opinion through library routines) on the tiny config
# ---------------------------------------------------------------------------------------------
def torch_decode_step(params, w, kv, tok, pos):
    """One decode step with torch float64 ops: F.rms_norm, SDPA with GQA, F.silu."""
    L, nq, nkv, hd = params["n_layers"], params["n_heads"], params["n_kv_heads"], params["head_dim"]
    eps, theta = params["rms_eps"], params["rope_theta"]

    def T(bits):
        return torch.from_numpy(np.asarray(bits).view(np.int16).copy()).view(torch.bfloat16).double()

    half = hd // 2
    inv = torch.tensor([theta ** (-2.0 * j / hd) for j in range(half)], dtype=torch.float64)
    c, s = torch.cos(pos * inv), torch.sin(pos * inv)

    def rope(x):
        a, b = x[..., :half], x[..., half:]
        return torch.cat([a * c - b * s, b * c + a * s], -1)

    r = T(w["embed"])[tok]
    kvt = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16)
    for l in range(L):
        lw = w["layers"][l]
        x = F.rms_norm(r, (r.shape[-1],), T(lw["attn_norm"]), eps)
        q = rope((x @ T(lw["wq"]).T).view(nq, hd))
        k = rope((x @ T(lw["wk"]).T).view(nkv, hd))
        v = (x @ T(lw["wv"]).T).view(nkv, hd)
        kvt[l, 0, 0, :, pos] = k.to(torch.bfloat16)
        kvt[l, 1, 0, :, pos] = v.to(torch.bfloat16)
        K = kvt[l, 0, 0, :, : pos + 1].double()
        V = kvt[l, 1, 0, :, : pos + 1].double()
        o = F.scaled_dot_product_attention(q[None, :, None, :], K[None], V[None],
                                           enable_gqa=True)[0, :, 0, :]
        r = r + o.reshape(-1) @ T(lw["wo"]).T
        x = F.rms_norm(r, (r.shape[-1],), T(lw["mlp_norm"]), eps)
        r = r + (F.silu(x @ T(lw["wg"]).T) * (x @ T(lw["wu"]).T)) @ T(lw["wd"]).T
    x = F.rms_norm(r, (r.shape[-1],), T(w["final_norm"]), eps)
    lm = w["lm_head"] if w["lm_head"] is not None else w["embed"]
    return (x @ T(lm).T).numpy()


def test_torch_second_opinion_tiny():
    cfg = synth.get_config("tiny")
    w = synth.make_weights(cfg, 0, random_gains=True)
    params, wn = synth.oracle_inputs(w)
    kv1 = np.zeros((cfg.n_layers, 2, 1, cfg.n_kv_heads, 8, cfg.head_dim), np.uint16)
    kv2 = kv1.copy()
    toks = synth.make_tokens(cfg, 0)[0, :6].numpy()
    dec = oracle.Decoder(params, wn)
    for p, t in enumerate(toks):
        a = dec.step(kv1, np.array([t]), p)[0]
        b = torch_decode_step(params, wn, kv2, int(t), p)
        assert np.max(np.abs(a - b)) < 1e-11
    assert np.array_equal(kv1, kv2)


def test_fp32_mode_close_to_fp64():
    cfg = synth.get_config("tiny")
    w = synth.make_weights(cfg, 0)
    params, wn = synth.oracle_inputs(w)
    toks = synth.make_tokens(cfg, 0)[0, :4].numpy()
    kv = np.zeros((2, 2, 1, 2, 8, 64), np.uint16)
    a = _incremental(params, wn, toks, kv.copy(), 0, np.float64)
    b = _incremental(params, wn, toks, kv.copy(), 0, np.float32)
    assert np.max(np.abs(a - b)) < 1e-4
