"""Prompt processing (amk_prefill), GPU only: a prompt run through the operator kernels up to 16
tokens at a time must leave the KV rows and the last token's logits that the oracle reaches by
feeding the prompt one token at a time, and the megakernel must decode on from that cache."""
import numpy as np
import pytest
import torch

import oracle
from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import LOGIT_TOL, MARGIN, kv_row_error, log, worst_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path,n_prompt,wtype", [("megakernel", 40, "bf16"), ("unfused", 40, "bf16"),
                                                 ("megakernel", 1, "bf16"), ("megakernel", 17, "bf16"),
                                                 ("megakernel", 33, "int8"), ("megakernel", 33, "int4")])
def test_prefill_then_decode_matches_oracle(path, n_prompt, wtype):
    cfg = synth.get_config("tiny").replace(prompt=0, prefill=0, steps=6, wtype=wtype)
    if wtype == "int4":
        cfg = cfg.replace(ffn=768, group=128)
    n_dec = 6
    max_seq = n_prompt + n_dec + 1
    w = synth.make_weights(cfg, 21)
    model = Model(cfg, w, path=path, max_seq=max_seq)
    kv = model.kv(1, max_seq)
    prompt = torch.from_numpy(
        np.random.default_rng(21).integers(0, cfg.vocab, n_prompt).astype(np.int32)).cuda()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    nxt = model.prefill(kv, prompt, 0, logits=logits)
    dec_logits = torch.empty((n_dec, 1, cfg.vocab), dtype=torch.float32, device="cuda")
    toks = model.steps(kv, nxt, n_prompt, n_dec, logits=dec_logits)
    model.sync()
    kv_dev = synth.bf16_to_numpy_bits(kv.tensor.cpu())

    params, wn = synth.oracle_inputs(w)
    dec = oracle.Decoder(params, wn)
    kv_np = np.zeros(kv_dev.shape, np.uint16)
    lo = None
    for i, t in enumerate(prompt.cpu().numpy()):
        lo = dec.step(kv_np, np.array([int(t)]), i)[0]
    worst = float(np.max(np.abs(logits.cpu().numpy() - lo)))
    assert worst <= LOGIT_TOL, worst
    if oracle.top2_margin(lo[None])[0] > MARGIN:
        assert int(nxt.item()) == oracle.argmax_lowest(lo[None])[0]
    assert kv_row_error(kv_dev[:, :, :, :, :n_prompt], kv_np[:, :, :, :, :n_prompt],
                        f"prefill/{path}/{wtype}/{n_prompt}") <= 1.0
    # decoding on from the prompt's cache, the oracle fed the device's tokens
    tok = int(nxt.item())
    g_toks, g_lo = toks.cpu().numpy(), dec_logits.cpu().numpy().astype(np.float64)
    for i in range(n_dec):
        lo = dec.step(kv_np, np.array([tok]), n_prompt + i)[0]
        worst = worst_of(worst, float(np.max(np.abs(g_lo[i, 0] - lo))))
        if oracle.top2_margin(lo[None])[0] > MARGIN:
            assert g_toks[i, 0] == oracle.argmax_lowest(lo[None])[0], i
        tok = int(g_toks[i, 0])
    log(f"prefill {path} n={n_prompt}: max_abs {worst:.2e}")
    assert worst <= LOGIT_TOL
    kv.close()
    model.close()


def test_prefill_into_one_sequence_of_a_batch():
    """A batch-2 model: the prompt goes to sequence 1 after a 5-position prefix; sequence 0's cache
    is untouched, and the logits match the oracle decoding sequence 1 alone."""
    cfg = synth.get_config("tiny").replace(batch=2, prompt=0, prefill=5, steps=1)
    max_seq = 5 + 20 + 1
    w = synth.make_weights(cfg, 22)
    kv_host = synth.make_kv(cfg, max_seq, 22)
    model = Model(cfg, w, max_seq=max_seq)
    kv = model.kv(2, max_seq)
    kv.tensor.copy_(kv_host.to(kv.tensor.device))
    prompt = torch.from_numpy(np.arange(20, dtype=np.int32) * 37 % cfg.vocab).cuda()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    model.prefill(kv, prompt, 5, seq=1, logits=logits)
    model.sync()
    kv_dev = synth.bf16_to_numpy_bits(kv.tensor.cpu())
    kv_np = synth.bf16_to_numpy_bits(kv_host).copy()
    assert np.array_equal(kv_dev[:, :, 0], kv_np[:, :, 0])
    params, wn = synth.oracle_inputs(w)
    dec = oracle.Decoder(params, wn)
    kv1 = kv_np[:, :, 1:2].copy()
    for i, t in enumerate(prompt.cpu().numpy()):
        lo = dec.step(kv1, np.array([int(t)]), 5 + i)[0]
    assert np.max(np.abs(logits.cpu().numpy() - lo)) <= LOGIT_TOL
    assert kv_row_error(kv_dev[:, :, 1:2, :, 5:25], kv1[:, :, :, :, 5:25], "prefill/seq1") <= 1.0
    assert np.array_equal(kv_dev[:, :, 1, :, :5], kv_np[:, :, 1, :, :5])
    kv.close()
    model.close()


def test_prefill_argument_errors():
    cfg = synth.get_config("tiny").replace(prompt=0, prefill=0, steps=1)
    model = Model(cfg, synth.make_weights(cfg, 1), max_seq=16)
    kv = model.kv(1, 16)
    p = torch.zeros(8, dtype=torch.int32, device="cuda")
    for kw, status in ((dict(pos0=9), _lib.AMK_E_CAPACITY), (dict(seq=1), _lib.AMK_E_CAPACITY),
                       (dict(pos0=-1), _lib.AMK_E_CAPACITY)):
        with pytest.raises(_lib.AmkError) as e:
            model.prefill(kv, p, **kw)
        assert e.value.status == status
    with pytest.raises(_lib.AmkError) as e:
        model.prefill(kv, p[:0])
    assert e.value.status == _lib.AMK_E_INVALID
    model.prefill(kv, p, 8)  # the last positions that fit
    model.sync()
    kv.close()
    model.close()
