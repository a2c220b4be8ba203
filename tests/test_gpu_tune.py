"""Profile-guided re-tiling on the device (amk_model_tune / amk_model_set_schedule), then the
tuned schedule checked against the oracle like any other (GPU only)."""
import pytest

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd import blob as B
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import assert_parity, log, teacher_forced

pytestmark = pytest.mark.gpu


def test_tuned_schedule_keeps_parity():
    cfg = synth.get_config("smollm2_135m")
    w = synth.make_weights(cfg, 6, threads=16)
    model = Model(cfg, w, max_seq=cfg.max_seq)
    kv = model.kv(1, cfg.max_seq)
    before = model.schedule()
    us = model.tune(kv, cfg.prefill, rounds=3, steps=2, gain=0.6)
    after = model.schedule()
    log(f"135m tuned: {us:.1f} us/step")
    assert us > 0
    assert _lib.schedule_validate(after)[0] == _lib.AMK_OK
    b0, b1 = B.Blob(before), B.Blob(after)
    assert b0.hdr.n_tasks == b1.hdr.n_tasks
    kv.close()
    rep = teacher_forced(cfg, "megakernel", seed=6, n_calls=3, weights=w, model=model)
    assert_parity(rep)
    # a schedule of another structure is refused and the model keeps working
    other = _lib.schedule_build(_lib.make_config(cfg, max_seq=cfg.max_seq), 1, model.info().n_cu,
                                _lib.amk_sched_params(attn_blocks=b1.hdr.attn_blocks + 1, search=0))
    with pytest.raises(_lib.AmkError) as e:
        model.set_schedule(other)
    assert e.value.status == _lib.AMK_E_UNSUPPORTED
    model.set_schedule(before)
    rep = teacher_forced(cfg, "megakernel", seed=6, n_calls=2, weights=w, model=model)
    assert_parity(rep)
    model.close()


def test_tuned_batched_schedule_keeps_the_weight_groups():
    """Re-tiling a model of batch capacity 4, whose weights are tile-major: the tuned GEMV tiles
    stay on the 16-row weight groups and the tuned model still matches the oracle."""
    cfg = synth.get_config("tiny").replace(batch=4)
    w = synth.make_weights(cfg, 9, threads=16)
    model = Model(cfg, w, max_seq=cfg.max_seq)
    kv = model.kv(cfg.batch, cfg.max_seq)
    us = model.tune(kv, 8, rounds=2, steps=2, gain=0.6)
    after = model.schedule()
    log(f"tiny batch-4 tuned: {us:.1f} us/step")
    assert us > 0
    assert _lib.schedule_validate(after)[0] == _lib.AMK_OK
    t = B.Blob(after).all_tasks()
    g = t[t["type"] == B.T_GEMV]
    assert (g["a0"] % 16 == 0).all()
    kv.close()
    rep = teacher_forced(cfg, "megakernel", seed=9, n_calls=10, weights=w, model=model)
    assert rep.tokens_checked > 0
    assert_parity(rep)
    model.close()
