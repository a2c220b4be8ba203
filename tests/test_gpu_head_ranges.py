"""Batch-1 schedules whose attention tasks cover a range of a KV group's query heads, against the
oracle: ranges of one head (one pass each), whole groups (one pass of all the group's heads) and,
for a group of three heads, the instance of four heads per pass running a range of three."""
import pytest
import torch

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import assert_parity, log, teacher_forced

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,heads,n_calls", [("tiny", 1, 12), ("tiny", 2, 12),
                                                ("smollm2_135m", 1, 4), ("smollm2_135m", 3, 4)])
def test_head_ranges_match_the_oracle(name, heads, n_calls):
    cfg = synth.get_config(name)
    qpg = cfg.n_heads // cfg.n_kv_heads
    max_seq = max(cfg.max_seq, cfg.first_pos + n_calls + 1)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    p = _lib.amk_sched_params(search=0, heads_per_task=heads, ctx_hint=cfg.first_pos + n_calls)
    blob = _lib.schedule_build(_lib.make_config(cfg, cfg.batch, max_seq), cfg.batch, n_cu, p)
    w = synth.make_weights(cfg, 0, threads=16)
    m = Model(cfg, w, path="megakernel", max_seq=max_seq, schedule=blob)
    try:
        info = m.info()
        want = 1 if heads == 1 else (2 if heads == 2 else 4)
        log(f"  [{name}] {qpg} heads per group, {heads} per task: instance of {info.heads_per_pass} "
            f"heads per pass, {info.n_tasks} tasks")
        assert info.heads_per_pass == want
        rep = teacher_forced(cfg, "megakernel", n_calls=n_calls, weights=w, model=m)
    finally:
        m.close()
    assert_parity(rep)
