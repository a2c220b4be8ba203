"""Greedy argmax ties on the GPU: two LM-head rows made identical give bit-identical logits, and
the lower index must win, as the oracle's argmax does (ties towards the lowest index), whether
the two rows fall in one LM tile or in different tiles (the tie is then decided by the combine
of the tiles' partial maxima)."""
import numpy as np
import pytest
import torch

import oracle
from persistent_decode_megakernel_amd import synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _duplicate_rows(w, src, dsts):
    lm = w.lm_head.clone()
    for d in dsts:
        lm[d] = lm[src]
    sc = None
    if w.lm_head_scale is not None:
        sc = w.lm_head_scale.clone()
        for d in dsts:
            sc[d] = sc[src]
    return synth.Weights(cfg=w.cfg, embed=w.embed, final_norm=w.final_norm, lm_head=lm,
                         lm_head_scale=sc, layers=w.layers, scales=w.scales,
                         attn_norm=w.attn_norm, mlp_norm=w.mlp_norm)


@pytest.mark.parametrize("name,path", [("tiny", "megakernel"), ("tiny", "unfused"),
                                       ("tiny_b3", "megakernel"), ("tiny_int8", "megakernel")])
@pytest.mark.parametrize("where", ["same_tile", "other_tile"])
def test_tied_logits_pick_the_lowest_index(name, path, where):
    base = synth.get_config("tiny").replace(prompt=0, prefill=12, steps=1)
    cfg = {"tiny": base, "tiny_b3": base.replace(batch=3),
           "tiny_int8": base.replace(wtype="int8")}[name]
    # a seed whose first step has a clear maximum for sequence 0 (so device rounding cannot move
    # the maximum to another row) at an index with room below it
    for seed in range(11, 40):
        w = synth.make_weights(cfg, seed, threads=16)
        kv_host = synth.make_kv(cfg, cfg.max_seq, seed)
        params, wn = synth.oracle_inputs(w)
        tok = synth.make_tokens(cfg, seed)[:, 0].numpy().astype(np.int64)
        lo = oracle.Decoder(params, wn).step(synth.bf16_to_numpy_bits(kv_host).copy(), tok,
                                             cfg.prefill)
        top = int(oracle.argmax_lowest(lo)[0])  # sequence 0's argmax
        if top >= 8 and oracle.top2_margin(lo)[0] > 0.05:
            break
    else:
        pytest.fail("no seed with a confident first step")
    # a lower-index copy of the top row (next to it, or a third of the vocabulary away), and a
    # higher-index copy
    low = top - 1 if where == "same_tile" else top // 3
    high = min(cfg.vocab - 1, top + 1) if where == "same_tile" else (top + cfg.vocab) // 2
    w2 = _duplicate_rows(w, top, [low, high] if high != top else [low])
    params2, wn2 = synth.oracle_inputs(w2)
    lo2 = oracle.Decoder(params2, wn2).step(synth.bf16_to_numpy_bits(kv_host).copy(), tok, cfg.prefill)
    assert lo2[0, low] == lo2[0, top] and int(oracle.argmax_lowest(lo2)[0]) == low
    model = Model(cfg, w2, path=path, max_seq=cfg.max_seq)
    kv = model.kv(cfg.batch, cfg.max_seq)
    kv.tensor.copy_(kv_host.to(kv.tensor.device))
    logits = torch.empty((cfg.batch, cfg.vocab), dtype=torch.float32, device="cuda")
    nxt = model.step(kv, torch.from_numpy(tok.astype(np.int32)).cuda(), cfg.prefill, logits)
    model.sync()
    g = logits.cpu().numpy()
    assert g[0, low] == g[0, top] == g[0, high], "duplicated rows gave different logits"
    assert int(np.argmax(g[0])) == low  # the duplicates are the maximum on the device too
    assert int(nxt[0].item()) == low, f"tie resolved to {int(nxt[0].item())}, expected {low}"
    log(f"{name}/{path}/{where}: rows {low}, {top}, {high} tie; next = {low}")
    kv.close()
    model.close()
