"""Determinism of the megakernel, GPU only.

* Graph capture: a megakernel step captured into a hipGraph and replayed reproduces the eager
  launches bit for bit, with eager steps and host synchronisations between replays. The step's
  epoch lives on the device, so each replay advances it like an eager launch does.
* Schedule invariance: two frozen schedules with the same decomposition (same tiles and KV blocks)
  but different task-to-CU placement give bitwise-identical tokens, logits and KV rows, also when
  the two models have run different numbers of steps before (different epochs)."""
import numpy as np
import pytest
import torch

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _cfg(name):
    tiny = synth.get_config("tiny").replace(prompt=0, prefill=24, steps=6)
    return {"tiny": tiny, "tiny_b3": tiny.replace(batch=3),
            "tiny_int8": tiny.replace(wtype="int8"),
            "smollm2_135m": synth.get_config("smollm2_135m").replace(prefill=40, steps=6)}[name]


@pytest.mark.parametrize("name", ["tiny", "tiny_b3", "tiny_int8"])
def test_megakernel_graph_replays_match_eager(name):
    cfg = _cfg(name)
    log(f"graph replay: {name}")
    w = synth.make_weights(cfg, 5, threads=16)
    max_seq = cfg.max_seq
    kv_host = synth.make_kv(cfg, max_seq, 5, threads=16)
    model = Model(cfg, w, path="megakernel", max_seq=max_seq)
    kv = model.kv(cfg.batch, max_seq)
    n, P, B = cfg.steps, cfg.prefill, cfg.batch
    first = synth.make_tokens(cfg, 5)[:, 0].to(torch.int32).cuda()
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty_like(tok)
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")

    def restart():
        kv.tensor.copy_(kv_host.to(kv.tensor.device))
        tok.copy_(first)

    restart()
    eager = []
    for i in range(n):
        model.step(kv, tok, P + i, logits, next_out=nxt)
        tok.copy_(nxt)
        model.sync()
        eager.append((logits.cpu().clone(), nxt.cpu().clone()))
    kv_eager = kv.tensor.cpu()

    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    graphs = []
    with torch.cuda.stream(cap):
        for i in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                model.step(kv, tok, P + i, logits, next_out=nxt)
                tok.copy_(nxt)
            graphs.append(g)
    stream.wait_stream(cap)
    torch.cuda.synchronize()

    for rep in range(3):
        restart()
        if rep == 1:
            # eager steps between replays (on a scratch cache): the device epoch moves on
            kv2 = model.kv(B, max_seq)
            t2 = first.clone()
            for i in range(3):
                model.step(kv2, t2, i, next_out=t2)
            model.sync()
            kv2.close()
        torch.cuda.synchronize()
        for i in range(n):
            graphs[i].replay()
            torch.cuda.synchronize()
            assert torch.equal(logits.cpu(), eager[i][0]), f"replay {rep} step {i}: logits differ"
            assert torch.equal(nxt.cpu(), eager[i][1]), f"replay {rep} step {i}: tokens differ"
        model.sync()
        assert torch.equal(kv.tensor.cpu(), kv_eager), f"replay {rep}: KV cache differs"
        log(f"  {name}: graph replay pass {rep}, {n} steps bit-identical to eager launches")
    del graphs
    kv.close()
    model.close()


def _run(cfg, w, kv_host, blob, pre_steps, n):
    """n greedy steps (one launch each) after pre_steps unrelated steps on a scratch cache."""
    max_seq = cfg.max_seq
    model = Model(cfg, w, path="megakernel", max_seq=max_seq, schedule=blob)
    B = cfg.batch
    first = synth.make_tokens(cfg, 9)[:, 0].to(torch.int32).cuda()
    if pre_steps:
        kv0 = model.kv(B, max_seq)
        t = first.clone()
        for i in range(pre_steps):
            model.step(kv0, t, i, next_out=t)
        model.sync()
        kv0.close()
    kv = model.kv(B, max_seq)
    kv.tensor.copy_(kv_host.to(kv.tensor.device))
    tok = first.clone()
    lg = torch.empty((n, B, cfg.vocab), dtype=torch.float32, device="cuda")
    ids = torch.empty((n, B), dtype=torch.int32, device="cuda")
    for i in range(n):
        model.step(kv, tok, cfg.prefill + i, lg[i], next_out=ids[i])
        tok = ids[i]
    model.sync()
    out = (lg.cpu(), ids.cpu(), kv.tensor.cpu())
    kv.close()
    model.close()
    return out


@pytest.mark.parametrize("name", ["tiny", "tiny_b3", "smollm2_135m"])
def test_schedule_placement_invariance(name):
    cfg = _cfg(name)
    log(f"schedule invariance: {name}")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    c = _lib.make_config(cfg, cfg.batch, cfg.max_seq)
    base = _lib.schedule_build(c, cfg.batch, n_cu, _lib.amk_sched_params(search=0))
    from persistent_decode_megakernel_amd import blob as B
    b0 = B.Blob(base)
    blocks = int(b0.hdr.attn_blocks)
    other = _lib.schedule_build(c, cfg.batch, n_cu, _lib.amk_sched_params(
        search=0, placement=1, rotate=1, attn_blocks=blocks))
    b1 = B.Blob(other)
    t0 = np.sort(b0.all_tasks(), order="id")
    t1 = np.sort(b1.all_tasks(), order="id")
    same = ("type", "mat", "layer", "a0", "a1", "w0_lo", "w0_hi", "w1_lo", "w1_hi")
    assert all(np.array_equal(t0[f], t1[f]) for f in same), "decompositions differ"
    cu0 = {int(t["id"]): c_ for c_, v in enumerate(b0.per_cu) for t in v}
    cu1 = {int(t["id"]): c_ for c_, v in enumerate(b1.per_cu) for t in v}
    moved = sum(cu0[i] != cu1[i] for i in cu0)
    assert moved > len(cu0) // 2, "placements hardly differ"
    w = synth.make_weights(cfg, 9, threads=16)
    kv_host = synth.make_kv(cfg, cfg.max_seq, 9, threads=16)
    n = cfg.steps
    a = _run(cfg, w, kv_host, base, 0, n)
    b = _run(cfg, w, kv_host, other, 3, n)
    assert torch.equal(a[1], b[1]), "tokens differ between placements"
    assert torch.equal(a[0], b[0]), "logits differ between placements"
    assert torch.equal(a[2], b[2]), "KV rows differ between placements"
    log(f"  {name}: {moved}/{len(cu0)} tasks on other CUs, {n} steps bit-identical")
