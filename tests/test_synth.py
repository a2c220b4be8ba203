"""Seeded synthetic inputs: determinism and distribution moments."""
import numpy as np
import torch

from persistent_decode_megakernel_amd import synth


def test_same_seed_same_bytes_and_order_independent():
    cfg = synth.get_config("tiny")
    a = synth.make_weights(cfg, 0, threads=1)
    b = synth.make_weights(cfg, 0, threads=4)
    for l in range(cfg.n_layers):
        for m in synth.MATS:
            assert torch.equal(a.layers[l][m], b.layers[l][m])
    c = synth.make_weights(cfg, 1)
    assert not torch.equal(a.layers[0]["wq"], c.layers[0]["wq"])
    assert torch.equal(synth.make_tokens(cfg, 0), synth.make_tokens(cfg, 0))


def test_moments_and_ranges():
    cfg = synth.get_config("tiny")
    w = synth.make_weights(cfg, 0)
    x = torch.cat([w.layers[l][m].float().flatten() for l in range(2) for m in synth.MATS])
    assert abs(x.mean().item()) < 2e-4 and abs(x.std().item() - 0.02) < 2e-4
    assert torch.all(w.attn_norm[0].float() == 1.0)
    t = synth.make_tokens(cfg, 0)
    assert t.shape == (1, 32) and t.dtype == torch.int32
    assert int(t.min()) >= 0 and int(t.max()) < cfg.vocab
    ci = synth.micro_config(L=1, d=256, F=512, V=300, wtype="int8")
    wi = synth.make_weights(ci, 0)
    q = wi.layers[0]["wg"]
    assert int(q.min()) == -127 and int(q.max()) == 127
    s = wi.scales[0]["wg"]
    assert float(s.min()) >= 1e-4 and float(s.max()) <= 4e-4
    kvc = synth.micro_config(L=1, d=64, nq=2, nkv=1, hd=32, F=96, V=128, prefill=500)
    kv = synth.make_kv(kvc, 510, 0).float()
    pre = kv[..., :500, :]
    assert abs(pre.mean().item()) < 0.02 and abs(pre.std().item() - 1.0) < 0.02
    assert torch.all(kv[..., 500:, :] == 0)


def test_config_shapes():
    c = synth.get_config("llama2_7b")
    total = sum(np.prod(s) for s in c.mat_shapes().values()) * c.n_layers + c.vocab * c.hidden
    assert total == 6_607_077_376
    c = synth.get_config("smollm2_135m")
    total = sum(np.prod(s) for s in c.mat_shapes().values()) * c.n_layers + c.vocab * c.hidden
    assert total == 134_479_872
    assert synth.get_config("tiny").n_calls == 47
