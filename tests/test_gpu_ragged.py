"""Sequences at different positions in one batched step (amk_decode_steps_ragged), GPU only: each
sequence's logits, tokens and appended KV rows against the oracle decoding that sequence alone at
its own positions (batch rows are independent, which the oracle's pins establish)."""
import numpy as np
import pytest
import torch

import oracle
from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import LOGIT_TOL, MARGIN, kv_row_error, log, worst_of

pytestmark = pytest.mark.gpu


def _run(cfg, path, pos0, n, seed, wtype_cfg=None):
    w = synth.make_weights(cfg, seed)
    max_seq = max(pos0) + n + 1
    kv_host = synth.make_kv(cfg, max_seq, seed)
    model = Model(cfg, w, path=path, max_seq=max_seq)
    kv = model.kv(cfg.batch, max_seq)
    kv.tensor.copy_(kv_host.to(kv.tensor.device))
    first = synth.make_tokens(cfg, seed)[:, 0].to(torch.int32).cuda()
    logits = torch.empty((n, cfg.batch, cfg.vocab), dtype=torch.float32, device="cuda")
    toks = model.steps(kv, first.clone(), list(pos0), n, logits=logits)
    model.sync()
    out = (w, kv_host, first.cpu().numpy(), toks.cpu().numpy(), logits.cpu().numpy().astype(np.float64),
           synth.bf16_to_numpy_bits(kv.tensor.cpu()))
    kv.close()
    model.close()
    return out


@pytest.mark.parametrize("path,batch,wtype", [("megakernel", 4, "bf16"), ("unfused", 4, "bf16"),
                                              ("megakernel", 1, "bf16"), ("megakernel", 11, "bf16"),
                                              ("megakernel", 5, "int8"), ("megakernel", 3, "int4")])
def test_ragged_positions_match_per_sequence_oracle(path, batch, wtype):
    cfg = synth.get_config("tiny").replace(batch=batch, prompt=0, prefill=24, steps=6, wtype=wtype)
    if wtype == "int4":
        cfg = cfg.replace(ffn=768, group=128)
    pos0 = [24 - (7 * b) % 23 for b in range(batch)]  # 24, 17, 10, 3, 19, ...
    n = 6
    w, kv_host, first, toks, logits, kv_dev = _run(cfg, path, pos0, n, seed=11)
    params, wn = synth.oracle_inputs(w)
    kv_np = synth.bf16_to_numpy_bits(kv_host).copy()
    worst, checked = 0.0, 0
    for b in range(batch):
        dec = oracle.Decoder(params, wn)
        kv_b = kv_np[:, :, b:b + 1].copy()
        tok = int(first[b])
        for i in range(n):
            lo = dec.step(kv_b, np.array([tok]), pos0[b] + i)[0]
            worst = worst_of(worst, float(np.max(np.abs(logits[i, b] - lo))))
            if oracle.top2_margin(lo[None])[0] > MARGIN:
                checked += 1
                assert toks[i, b] == oracle.argmax_lowest(lo[None])[0], (b, i)
            tok = int(toks[i, b])
        # the rows this sequence appended, within the KV-row bound of the oracle's
        rows = slice(pos0[b], pos0[b] + n)
        assert kv_row_error(kv_dev[:, :, b, :, rows, :], kv_b[:, :, 0, :, rows, :],
                            f"ragged/{path}/B{batch}/seq{b}") <= 1.0, b
        # nothing else of the sequence's cache changed
        other = np.ones(kv_dev.shape[4], bool)
        other[rows] = False
        assert np.array_equal(kv_dev[:, :, b, :, other, :], kv_np[:, :, b, :, other, :]), b
    log(f"ragged {path} B={batch}: max_abs {worst:.2e}, {checked} confident tokens")
    assert worst <= LOGIT_TOL
    assert checked > 0


def test_ragged_equals_uniform_when_positions_agree():
    """The ragged entry point with equal positions is the plain multi-step call, bit for bit."""
    cfg = synth.get_config("tiny").replace(batch=3, prompt=0, prefill=16, steps=4)
    a = _run(cfg, "megakernel", [16, 16, 16], 4, seed=12)
    w = synth.make_weights(cfg, 12)
    max_seq = 16 + 4 + 1
    kv_host = synth.make_kv(cfg, max_seq, 12)
    model = Model(cfg, w, max_seq=max_seq)
    kv = model.kv(3, max_seq)
    kv.tensor.copy_(kv_host.to(kv.tensor.device))
    first = synth.make_tokens(cfg, 12)[:, 0].to(torch.int32).cuda()
    logits = torch.empty((4, 3, cfg.vocab), dtype=torch.float32, device="cuda")
    toks = model.steps(kv, first, 16, 4, logits=logits)
    model.sync()
    assert np.array_equal(a[3], toks.cpu().numpy())
    assert np.array_equal(a[4], logits.cpu().numpy().astype(np.float64))
    kv.close()
    model.close()


def test_ragged_capacity_errors():
    cfg = synth.get_config("tiny").replace(batch=2, prompt=0, prefill=4, steps=2)
    w = synth.make_weights(cfg, 1)
    model = Model(cfg, w, max_seq=10)
    kv = model.kv(2, 10)
    tok = torch.zeros(2, dtype=torch.int32, device="cuda")
    for bad in ([0, 9], [-1, 3]):
        with pytest.raises(_lib.AmkError) as e:
            model.steps(kv, tok, bad, 2)
        assert e.value.status == _lib.AMK_E_CAPACITY
    out = model.steps(kv, tok, [0, 7], 2)  # the largest legal positions still run
    model.sync()
    assert out.shape == (2, 2)
    kv.close()
    model.close()
