"""The entry point that allocates nothing (amk_decode_steps_noalloc), GPU only: the same tokens,
logits and KV rows, bit for bit, as amk_decode_steps on the same model and inputs, on two calls
in a row (the second with a smaller input: fewer sequences, fewer steps, an earlier position),
with the static array left dirty by the calls before; and the refusal of a model whose step
scratch exceeds the array."""
import pytest
import torch

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _cfg(name):
    tiny = synth.get_config("tiny").replace(prompt=0, prefill=30, steps=9)
    return {
        "tiny_megakernel": (tiny, "megakernel"),
        "tiny_b4_megakernel": (tiny.replace(batch=4), "megakernel"),
        "tiny_int8_megakernel": (tiny.replace(wtype="int8"), "megakernel"),
        "tiny_b4_unfused": (tiny.replace(batch=4), "unfused"),
        "smollm2_135m_megakernel": (synth.get_config("smollm2_135m").replace(prefill=64, steps=9),
                                    "megakernel"),
    }[name]


def _call(model, cfg, kv_host, batch, pos, n, noalloc):
    """n steps of `batch` sequences from position pos on a fresh copy of the prefilled cache."""
    kv = model.kv(cfg.batch, cfg.max_seq)
    kv.tensor.copy_(kv_host.to(kv.tensor.device))
    first = synth.make_tokens(cfg, 3)[:batch, 0].to(torch.int32).cuda()
    logits = torch.full((n, batch, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((n, batch), -1, dtype=torch.int32, device="cuda")
    if noalloc:
        model.steps_noalloc(kv, first, pos, n, logits=logits, out=out)
    else:
        model.steps(kv, first, pos, n, logits=logits, out=out)
    model.sync()
    res = (out.cpu(), logits.cpu(), kv.tensor.cpu())
    kv.close()
    return res


@pytest.mark.parametrize("name", ["tiny_megakernel", "tiny_b4_megakernel", "tiny_int8_megakernel",
                                  "tiny_b4_unfused", "smollm2_135m_megakernel"])
def test_noalloc_matches_decode_steps(name):
    cfg, path = _cfg(name)
    log(f"noalloc: {name}")
    w = synth.make_weights(cfg, 3, threads=16)
    kv_host = synth.make_kv(cfg, cfg.max_seq, 3, threads=16)
    model = Model(cfg, w, path=path, max_seq=cfg.max_seq)
    assert model.info().scratch_bytes <= _lib.AMK_STATIC_SCRATCH_BYTES
    B, P = cfg.batch, cfg.prefill
    calls = [(B, P, 9), (max(1, B - 2), P - 20, 4)]  # the second call: a smaller input
    for i, (batch, pos, n) in enumerate(calls):
        ref = _call(model, cfg, kv_host, batch, pos, n, noalloc=False)
        got = _call(model, cfg, kv_host, batch, pos, n, noalloc=True)
        assert torch.equal(got[0], ref[0]), f"call {i}: tokens differ"
        assert torch.equal(got[1], ref[1]), f"call {i}: logits differ"
        assert torch.equal(got[2], ref[2]), f"call {i}: KV cache differs"
        log(f"  {name} call {i}: batch {batch}, {n} steps from {pos}: identical")
    # a second model's call in between leaves the array dirty; this model's call still matches
    other = Model(cfg, synth.make_weights(cfg, 4, threads=16), path=path, max_seq=cfg.max_seq)
    _call(other, cfg, kv_host, B, P, 3, noalloc=True)
    other.close()
    batch, pos, n = calls[1]
    ref = _call(model, cfg, kv_host, batch, pos, n, noalloc=False)
    got = _call(model, cfg, kv_host, batch, pos, n, noalloc=True)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])
    model.close()


def test_noalloc_refuses_a_model_beyond_the_array():
    # 2048 KV blocks per head at batch capacity 16: the attention partials alone exceed 64 MiB
    cfg = synth.get_config("tiny").replace(prompt=0, prefill=8, steps=2, batch=16)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    c = _lib.make_config(cfg, 16, cfg.max_seq)
    blob = _lib.schedule_build(c, 16, n_cu, _lib.amk_sched_params(search=0, attn_blocks=2048))
    model = Model(cfg, synth.make_weights(cfg, 3, threads=16), path="megakernel",
                  max_seq=cfg.max_seq, schedule=blob)
    assert model.info().scratch_bytes > _lib.AMK_STATIC_SCRATCH_BYTES
    kv = model.kv(16, cfg.max_seq)
    tok = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.AmkError) as e:
        model.steps_noalloc(kv, tok, 0, 1)
    assert e.value.status == _lib.AMK_E_CAPACITY
    kv.close()
    model.close()
