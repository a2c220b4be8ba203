"""Several greedy decode steps in one launch (amk_decode_steps), GPU only: checked against the
oracle replaying the device's own tokens, and against the same steps run one launch each (same
kernels, same inputs: identical tokens and logits)."""
import numpy as np
import pytest
import torch

import oracle
from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import LOGIT_TOL, MARGIN, log, worst_of

pytestmark = pytest.mark.gpu


def _setup(cfg, seed, path="megakernel", extra=0):
    w = synth.make_weights(cfg, seed, threads=16)
    max_seq = cfg.prefill + cfg.n_calls + 1 + extra
    kv_host = synth.make_kv(cfg, max_seq, seed, threads=16)
    model = Model(cfg, w, path=path, max_seq=max_seq)
    return w, kv_host, model, max_seq


def _fresh_kv(model, cfg, kv_host, max_seq):
    kv = model.kv(cfg.batch, max_seq)
    kv.tensor.copy_(kv_host.to(kv.tensor.device))
    return kv


@pytest.mark.parametrize("name,path", [("smollm2_135m", "megakernel"), ("tiny_b3", "megakernel"),
                                       ("tiny_b3", "unfused"), ("tiny_int8", "megakernel"),
                                       ("tiny_int4", "megakernel"), ("tiny_int4_b3", "megakernel")])
def test_multistep_equals_single_steps_and_oracle(name, path):
    tiny = synth.get_config("tiny").replace(prompt=0, prefill=20, steps=8)
    if name == "tiny_b3":
        cfg = tiny.replace(batch=3)
    elif name == "tiny_int8":
        cfg = tiny.replace(wtype="int8")
    elif name == "tiny_int4":
        cfg = tiny.replace(wtype="int4", ffn=768, group=128)
    elif name == "tiny_int4_b3":
        cfg = tiny.replace(wtype="int4", ffn=768, group=128, batch=3)
    else:
        cfg = synth.get_config(name)
    # n = 7: epochs of the two runs differ in their low bits, which batch-1 hand-off words carry
    # as tags; values are read with the tag bits cleared, so the runs still agree bit for bit
    n = 7
    w, kv_host, model, max_seq = _setup(cfg, 7, path)
    V, B, P = cfg.vocab, cfg.batch, cfg.prefill
    first = synth.make_tokens(cfg, 7)[:, 0].to(torch.int32).cuda()

    # one launch, n steps
    kv = _fresh_kv(model, cfg, kv_host, max_seq)
    logits_m = torch.empty((n, B, V), dtype=torch.float32, device="cuda")
    toks_m = model.steps(kv, first.clone(), P, n, logits=logits_m)
    model.sync()
    kv_m = kv.tensor.cpu()
    kv.close()

    # n launches of one step, tokens chained on the device
    kv = _fresh_kv(model, cfg, kv_host, max_seq)
    tok = first.clone()
    logits_s = torch.empty((n, B, V), dtype=torch.float32, device="cuda")
    toks_s = torch.empty((n, B), dtype=torch.int32, device="cuda")
    for i in range(n):
        model.step(kv, tok, P + i, logits=logits_s[i], next_out=toks_s[i])
        tok = toks_s[i]
    model.sync()
    kv_s = kv.tensor.cpu()
    kv.close()
    assert torch.equal(toks_m.cpu(), toks_s.cpu())
    assert torch.equal(logits_m.cpu(), logits_s.cpu())
    assert torch.equal(kv_m, kv_s)

    # the oracle, fed the device's tokens
    params, wn = synth.oracle_inputs(w)
    dec = oracle.Decoder(params, wn, dtype=np.float32 if cfg.n_layers > 2 else np.float64)
    kv_np = synth.bf16_to_numpy_bits(kv_host).copy()
    tok_np = first.cpu().numpy().astype(np.int64)
    g_toks = toks_m.cpu().numpy()
    g_logits = logits_m.cpu().numpy().astype(np.float64)
    worst, checked = 0.0, 0
    for i in range(n):
        lo = dec.step(kv_np, tok_np, P + i)
        worst = worst_of(worst, float(np.max(np.abs(g_logits[i] - lo))))
        ids, marg = oracle.argmax_lowest(lo), oracle.top2_margin(lo)
        for b in range(B):
            if marg[b] > MARGIN:
                checked += 1
                assert g_toks[i, b] == ids[b], (i, b, g_toks[i, b], ids[b], marg[b])
        tok_np = g_toks[i].astype(np.int64)
    log(f"{name}/{path} multistep: max_abs {worst:.2e}, {checked} confident tokens")
    assert worst <= LOGIT_TOL
    assert checked > 0
    model.close()


def test_multistep_capacity_and_arguments():
    cfg = synth.get_config("tiny").replace(prompt=0, prefill=4, steps=4)
    w, kv_host, model, max_seq = _setup(cfg, 1)
    kv = _fresh_kv(model, cfg, kv_host, max_seq)
    tok = synth.make_tokens(cfg, 1)[:, 0].to(torch.int32).cuda()
    with pytest.raises(_lib.AmkError) as e:
        model.steps(kv, tok, max_seq - 2, 3)
    assert e.value.status == _lib.AMK_E_CAPACITY
    with pytest.raises(_lib.AmkError) as e:
        model.steps(kv, tok, 0, 0)
    assert e.value.status == _lib.AMK_E_INVALID
    # the model still works after the refused calls
    out = model.steps(kv, tok, cfg.prefill, max_seq - cfg.prefill)
    model.sync()
    assert out.shape == (max_seq - cfg.prefill, 1)
    kv.close()
    model.close()
