"""Model creation caches the schedules it builds (GPU only): the first creation writes the built
blob, a later one with the same key reads it back (a different valid blob planted under that key
is what the model then runs), an invalid cached blob is rebuilt and replaced, and
AMK_CACHE_DIR=off writes nothing."""
import glob
import os

import pytest
import torch

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd.model import Model

pytestmark = pytest.mark.gpu


def test_schedule_cache(tmp_path, monkeypatch):
    cfg = synth.get_config("tiny").replace(prompt=0, prefill=8, steps=2)
    w = synth.make_weights(cfg, 3, threads=16)
    monkeypatch.setenv("AMK_CACHE_DIR", str(tmp_path))
    a = Model(cfg, w, max_seq=cfg.max_seq)
    files = glob.glob(str(tmp_path / "schedule-*.amks"))
    assert len(files) == 1
    built = a.schedule()
    assert open(files[0], "rb").read() == built
    a.close()
    # a different valid schedule of the same configuration under the key: it is what runs
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    other = _lib.schedule_build(_lib.make_config(cfg, cfg.batch, cfg.max_seq), cfg.batch, n_cu,
                                _lib.amk_sched_params(search=0, placement=1, rotate=1))
    assert other != built
    open(files[0], "wb").write(other)
    b = Model(cfg, w, max_seq=cfg.max_seq)
    assert b.schedule() == other
    kv = b.kv()
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    b.step(kv, tok, 0)
    b.sync()
    kv.close()
    b.close()
    # an invalid cached blob is rebuilt and replaced
    open(files[0], "wb").write(b"not a schedule")
    c = Model(cfg, w, max_seq=cfg.max_seq)
    assert c.schedule() == built
    assert open(files[0], "rb").read() == built
    c.close()
    # disabled
    monkeypatch.setenv("AMK_CACHE_DIR", "off")
    os.remove(files[0])
    Model(cfg, w, max_seq=cfg.max_seq).close()
    assert not glob.glob(str(tmp_path / "schedule-*.amks"))
