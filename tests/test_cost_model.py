"""The schedule search's cost model (host only): the calibrated model stored as JSON is the one
used when the caller passes none, for the CU count it was measured on; other counts, a missing or
incomplete file, or AMK_COST_MODEL=off fall back to the built-in values; and the makespan model
responds to its parameters as the kernel's overlap implies."""
import json
import os

import pytest

from persistent_decode_megakernel_amd import _lib, synth

FIT = {"cu_stream_gbs": 21.5, "hop_us": 3.25, "l2_gbs": 61.0, "task_us": 0.0, "prefetch_kb": 96.0}


@pytest.fixture
def model_file(tmp_path, monkeypatch):
    p = tmp_path / "cm.json"
    p.write_text(json.dumps({"n_cu": 256, "stream": [], "relay": [], "fit": FIT}))
    monkeypatch.setenv("AMK_COST_MODEL", str(p))
    return p


def test_calibrated_file_is_the_default(libamk, model_file):
    cm, src = _lib.cost_model_default(256)
    assert src == str(model_file)
    for k, v in FIT.items():
        assert getattr(cm, k) == pytest.approx(v)
    cm80, src80 = _lib.cost_model_default(80)  # measured on another CU count: not used
    assert src80 == "built-in" and cm80.hop_us != FIT["hop_us"]


@pytest.mark.parametrize("text", ["", "{", '{"n_cu": 256}', '{"n_cu": 256, "fit": {"hop_us": 1}}'])
def test_incomplete_files_are_ignored(libamk, tmp_path, monkeypatch, text):
    p = tmp_path / "bad.json"
    p.write_text(text)
    monkeypatch.setenv("AMK_COST_MODEL", str(p))
    assert _lib.cost_model_default(256)[1] == "built-in"


def test_off_and_missing(libamk, monkeypatch, tmp_path):
    monkeypatch.setenv("AMK_COST_MODEL", "off")
    assert _lib.cost_model_default(256)[1] == "built-in"
    monkeypatch.setenv("AMK_COST_MODEL", str(tmp_path / "absent.json"))
    assert _lib.cost_model_default(256)[1] == "built-in"


def test_committed_calibration_parses(libamk, monkeypatch):
    """The model measured on MI355X and shipped beside the library (if present) is complete."""
    monkeypatch.delenv("AMK_COST_MODEL", raising=False)
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "cost_model.json")
    if not os.path.exists(path):
        pytest.skip("no calibration shipped")
    rec = json.load(open(path))
    cm, src = _lib.cost_model_default(int(rec["n_cu"]))
    assert src == path
    assert cm.cu_stream_gbs == pytest.approx(rec["fit"]["cu_stream_gbs"])


def test_makespan_responds_to_the_model(libamk, monkeypatch):
    monkeypatch.setenv("AMK_COST_MODEL", "off")
    cfg = synth.get_config("llama2_7b")
    c = _lib.make_config(cfg, 1, 2113)
    blob = _lib.schedule_build(c, 1, 256, _lib.amk_sched_params(search=0))
    base = dict(cu_stream_gbs=28.0, hop_us=3.0, task_us=0.5, l2_gbs=80.0, prefetch_kb=128.0)

    def pred(**kw):
        d = dict(base, **kw)
        return _lib.schedule_predict(blob, 2081, _lib.amk_cost_model(**d))

    t = pred()
    assert pred(cu_stream_gbs=20.0) > t > pred(cu_stream_gbs=40.0)  # bandwidth bound
    assert pred(hop_us=6.0) > t                                       # each hop on the path
    assert pred(prefetch_kb=1e-6) > t                                  # prefetch hides part of a hop
    # the weights alone bound it from below: 13.2 GB over 256 CUs at 28 GB/s each
    assert t > 13.2e9 / (256 * 28e3)


@pytest.mark.parametrize("name", ["smollm2_135m", "llama2_7b"])
def test_fit_recovers_a_simulated_step(libamk, monkeypatch, name):
    """amk_schedule_predict_trace writes the model's own timeline as a task trace; fitting that
    trace gives back the fixed costs it was simulated with (every GEMV tile and attention block
    takes exactly task_us / attn_us beyond its terms) and a hop whose simulated step equals the
    traced one. A fit that mixed up the stamps, the byte counts or the prefetch rule would not."""
    monkeypatch.setenv("AMK_COST_MODEL", "off")
    cfg = synth.get_config(name)
    ctx = cfg.prefill + 9
    c = _lib.make_config(cfg, 1, cfg.prefill + 64)
    blob = _lib.schedule_build(c, 1, 256, _lib.amk_sched_params(search=0, ctx_hint=ctx))
    truth = _lib.amk_cost_model(cu_stream_gbs=27.0, hop_us=3.5, task_us=2.25, l2_gbs=20.0,
                                prefetch_kb=128.0, attn_us=6.5)
    tr = _lib.schedule_predict_trace(blob, ctx, truth)
    span = (tr[3:4 * (len(tr) // 4):4].max() - tr[0:4 * (len(tr) // 4):4].min()) * 0.01
    assert span == pytest.approx(_lib.schedule_predict(blob, ctx, truth), abs=0.02)
    base = _lib.amk_cost_model(cu_stream_gbs=27.0, l2_gbs=20.0, prefetch_kb=128.0)
    cm, rep = _lib.cost_model_fit(blob, tr[None, :], ctx, base)
    assert cm.task_us == pytest.approx(2.25, abs=0.02)
    assert cm.attn_us == pytest.approx(6.5, abs=0.1)
    assert cm.hop_us == pytest.approx(3.5, abs=0.05)
    assert rep["predicted_us"] == pytest.approx(rep["measured_us"], rel=1e-3)
    assert rep["fit"]["hop_us"] == pytest.approx(cm.hop_us, abs=1e-3)


def test_fit_rejects_bad_input(libamk):
    cfg = synth.get_config("tiny")
    c = _lib.make_config(cfg, 1, 64)
    blob = _lib.schedule_build(c, 1, 16, _lib.amk_sched_params(search=0))
    import numpy as np
    with pytest.raises(RuntimeError):
        _lib.cost_model_fit(blob, np.zeros((0, 8), np.uint64), 40)
    with pytest.raises(RuntimeError):
        _lib.cost_model_fit(blob[:100], np.zeros((1, 8), np.uint64), 40)
