"""Oracle parity at Llama-2-7B width (hidden 4096, 32 heads of 128, FFN 11008, vocab 32000) on a
two-layer model, GPU only. Every kernel runs at its full-size shapes (head_dim 128 attention over
several KV blocks, GEMVs with K = 4096 and 11008, a 32000-row LM head) while the float64 oracle
still follows each step:

* the unfused one-kernel-per-operator path (the ablation the megakernel is measured against) and
  the megakernel, teacher-forced, bf16 and W8A16;
* prompt processing (amk_prefill) of a 64-token prompt from an empty cache, then 12 greedy
  megakernel steps in one launch: the input-64 / output-12 workload of the pages' experiments,
  against the oracle fed the prompt token by token and then the device's own tokens."""
import numpy as np
import pytest
import torch

import oracle
from persistent_decode_megakernel_amd import synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import LOGIT_TOL, MARGIN, assert_parity, kv_row_error, log, teacher_forced, worst_of

pytestmark = pytest.mark.gpu

NAMES = ["llama2_7b_2l", "llama2_7b_2l_w8a16"]


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("path", ["unfused", "megakernel"])
def test_full_width_teacher_forced(name, path):
    cfg = synth.get_config(name)
    log(f"full width teacher-forced: {name}/{path}")
    rep = teacher_forced(cfg, path, seed=0)
    log(f"  {name}/{path}: {rep}")
    assert rep.steps == cfg.steps and rep.tokens_checked > 0
    assert_parity(rep)


@pytest.mark.parametrize("name", NAMES)
def test_full_width_prompt_then_decode(name):
    cfg = synth.get_config(name).replace(prefill=0)
    n_in, n_out = 64, 12
    max_seq = n_in + n_out + 1
    log(f"full width prompt {n_in} + {n_out} steps: {name}")
    w = synth.make_weights(cfg, 1, threads=16)
    model = Model(cfg, w, path="megakernel", max_seq=max_seq)
    kv = model.kv(1, max_seq)
    prompt = torch.from_numpy(
        np.random.default_rng(64).integers(0, cfg.vocab, n_in).astype(np.int32)).cuda()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    nxt = model.prefill(kv, prompt, 0, logits=logits)
    dec_logits = torch.empty((n_out, 1, cfg.vocab), dtype=torch.float32, device="cuda")
    toks = model.steps(kv, nxt, n_in, n_out, logits=dec_logits)
    model.sync()
    kv_dev = synth.bf16_to_numpy_bits(kv.tensor.cpu())

    params, wn = synth.oracle_inputs(w)
    dec = oracle.Decoder(params, wn)
    kv_np = np.zeros(kv_dev.shape, np.uint16)
    lo = None
    for i, t in enumerate(prompt.cpu().numpy()):
        lo = dec.step(kv_np, np.array([int(t)]), i)[0]
    worst = float(np.max(np.abs(logits.cpu().numpy() - lo)))
    checked = 0
    if oracle.top2_margin(lo[None])[0] > MARGIN:
        checked += 1
        assert int(nxt.item()) == oracle.argmax_lowest(lo[None])[0]
    assert kv_row_error(kv_dev[..., :n_in, :], kv_np[..., :n_in, :], f"{name}/prompt") <= 1.0
    tok = int(nxt.item())
    g_toks, g_lo = toks.cpu().numpy(), dec_logits.cpu().numpy().astype(np.float64)
    for i in range(n_out):
        lo = dec.step(kv_np, np.array([tok]), n_in + i)[0]
        worst = worst_of(worst, float(np.max(np.abs(g_lo[i, 0] - lo))))
        if oracle.top2_margin(lo[None])[0] > MARGIN:
            checked += 1
            assert g_toks[i, 0] == oracle.argmax_lowest(lo[None])[0], i
        tok = int(g_toks[i, 0])
    assert kv_row_error(kv_dev[..., n_in:n_in + n_out, :], kv_np[..., n_in:n_in + n_out, :],
                        f"{name}/decode") <= 1.0
    log(f"  {name}: prompt + decode max_abs {worst:.2e}, {checked} confident tokens")
    assert worst <= LOGIT_TOL
    assert checked >= 6
    kv.close()
    model.close()
