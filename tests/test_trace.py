"""Task-trace summaries and the Chrome/Perfetto export (host only), on the cost model's own
simulated timeline of real schedules (amk_schedule_predict_trace), whose totals are known."""
import json

import numpy as np
import pytest

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd import trace as T
from persistent_decode_megakernel_amd.blob import Blob

COST = dict(cu_stream_gbs=27.0, hop_us=3.0, task_us=1.5, l2_gbs=60.0, prefetch_kb=128.0, attn_us=4.0)


def _sim(name, batch=1, n_cu=64):
    cfg = synth.get_config(name)
    ctx = cfg.prefill + 1
    c = _lib.make_config(cfg, batch, cfg.prefill + 8)
    blob = _lib.schedule_build(c, batch, n_cu, _lib.amk_sched_params(search=0, ctx_hint=ctx))
    cm = _lib.amk_cost_model(**COST)
    return cfg, Blob(blob), _lib.schedule_predict_trace(blob, ctx, cm), _lib.schedule_predict(blob, ctx, cm)


@pytest.mark.parametrize("name,batch", [("tiny", 1), ("tiny", 3), ("smollm2_135m", 1)])
def test_summary_accounts_for_every_task(libamk, monkeypatch, name, batch):
    monkeypatch.setenv("AMK_COST_MODEL", "off")
    cfg, b, tr, span = _sim(name, batch)
    s = T.summarize(b, tr)
    assert s["step_us"] == pytest.approx(span, abs=0.05)
    ph = s["phases"]
    # five phases per layer (QKV, attention, O, gate/up, down), then the LM head and the argmax
    assert len(ph) == 5 * cfg.n_layers + 2
    assert sum(p["tasks"] for p in ph.values()) == b.hdr.n_tasks
    nblk = int(b.hdr.attn_blocks)
    qpg = cfg.n_heads // cfg.n_kv_heads
    ranges = {qpg // int(t["aux3"]) for v in b.per_cu for t in v if t["type"] == 2}.pop()
    for l in range(cfg.n_layers):
        assert ph[f"{l}:attn"]["tasks"] == cfg.n_kv_heads * ranges * nblk
        # every phase of a layer starts no earlier than the previous phase's first task starts
        assert ph[f"{l}:o"]["last_end_us"] > ph[f"{l}:attn"]["first_start_us"]
    assert ph[f"{10 ** 6}:argmax"]["tasks"] == 1
    assert ph[f"{10 ** 6}:argmax"]["last_end_us"] == pytest.approx(s["step_us"], abs=0.05)
    for p in ph.values():
        assert p["span_us"] >= 0 and p["wait_mean_us"] >= 0 and p["body_mean_us"] >= 0
        assert p["last_end_us"] <= s["step_us"] + 1e-6
    assert set(s["by_kind_mean_us"]) == {"qkv", "attn", "o", "gateup", "down", "lm_head", "argmax"}


def test_chrome_export(libamk, monkeypatch, tmp_path):
    monkeypatch.setenv("AMK_COST_MODEL", "off")
    cfg, b, tr, span = _sim("tiny")
    path = tmp_path / "trace.json"
    T.to_chrome_json(b, tr, str(path))
    ev = json.load(open(path))["traceEvents"]
    assert len(ev) == 2 * b.hdr.n_tasks  # a wait and a body per task
    n_cu = int(b.hdr.n_cu)
    for e in ev:
        assert e["ph"] == "X" and 0 <= e["tid"] < n_cu
        assert e["ts"] >= 0 and e["dur"] >= 0
        assert e["ts"] + e["dur"] <= span + 0.05
    # each CU's events do not overlap: a CU runs its tasks one after another
    by_cu = {}
    for e in ev:
        by_cu.setdefault(e["tid"], []).append((e["ts"], e["ts"] + e["dur"]))
    for spans in by_cu.values():
        spans.sort()
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert b0 >= a1 - 0.011
