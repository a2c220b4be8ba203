"""Profile-guided re-tiling of a frozen schedule (host only): synthetic task traces in which the
CUs stream at known, different rates; the rebalanced tiles must equalise the predicted finish
times of every GEMV phase, keep the schedule valid, and leave a balanced schedule unchanged."""
import numpy as np
import pytest

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd import blob as B


def _tiny_blob(n_cu=8, batch=1):
    cfg = synth.get_config("tiny")
    return _lib.schedule_build(_lib.make_config(cfg, max_batch=batch), batch, n_cu)


def _gemv_tasks(b: B.Blob):
    """[(id, cu, mat, layer, a0, a1)] of the GEMV tasks."""
    out = []
    for cu, v in enumerate(b.per_cu):
        for t in v:
            if t["type"] == B.T_GEMV:
                out.append((int(t["id"]), cu, int(t["mat"]), int(t["layer"]), int(t["a0"]), int(t["a1"])))
    return out


def _trace(b: B.Blob, us_per_row, start_us=None):
    """One step's trace: every GEMV tile staged at start_us[cu] (0 by default) and streaming
    us_per_row[cu] microseconds per row; stamps in 100 MHz ticks."""
    n = b.hdr.n_tasks
    tr = np.zeros(4 * n + b.hdr.n_cu, dtype=np.uint64)
    for tid, cu, mat, layer, a0, a1 in _gemv_tasks(b):
        st = 1000 + (0 if start_us is None else int(round(start_us[cu] * 100)))
        tr[4 * tid: 4 * tid + 4] = [st - 50, st - 10, st, st + int(round((a1 - a0) * us_per_row[cu] * 100))]
    return tr


def _finish_spread(b: B.Blob, us_per_row, start_us):
    """Largest spread (us) of predicted tile finish times over the GEMV phases."""
    phases = {}
    for tid, cu, mat, layer, a0, a1 in _gemv_tasks(b):
        phases.setdefault((mat, layer), []).append(start_us[cu] + (a1 - a0) * us_per_row[cu])
    return max(max(v) - min(v) for v in phases.values())


def test_balanced_schedule_is_a_fixed_point(libamk):
    blob = _tiny_blob()
    b = B.Blob(blob)
    tr = _trace(b, np.full(8, 0.05))
    # tiles of one phase have (nearly) equal rows and equal rates: nothing to move
    out = B.Blob(_lib.schedule_rebalance(blob, tr[None], gain=1.0))
    before = {t[0]: (t[4], t[5]) for t in _gemv_tasks(b)}
    after = {t[0]: (t[4], t[5]) for t in _gemv_tasks(out)}
    moved = sum(abs(after[k][0] - before[k][0]) for k in before)
    assert moved <= 2 * len(before), moved  # at most rounding to the row alignment


@pytest.mark.parametrize("n_cu", [8, 13])
def test_unequal_rates_are_equalised(libamk, n_cu):
    """Half of the CUs stream at half the rate and some start late: with gain 1 the predicted
    finish times of every phase agree to within the row alignment."""
    blob = _tiny_blob(n_cu)
    b = B.Blob(blob)
    rng = np.random.default_rng(0)
    rate = np.where(np.arange(n_cu) % 2 == 0, 0.02, 0.04)  # us per row
    start = rng.uniform(0.0, 1.0, n_cu)
    spread0 = _finish_spread(b, rate, start)
    out_blob = _lib.schedule_rebalance(blob, _trace(b, rate, start)[None], gain=1.0)
    out = B.Blob(out_blob)
    assert _lib.schedule_validate(out_blob)[0] == _lib.AMK_OK
    assert _lib.schedule_simulate(out_blob)[0] == _lib.AMK_OK
    spread1 = _finish_spread(out, rate, start)
    # each boundary rounds to the row alignment (2): a tile may be off by one pair, two tiles
    # in opposite directions
    assert spread1 < 0.1 * spread0 and spread1 <= 2 * 2 * 0.04 + 1e-9, (spread0, spread1)
    # ids, placement and the row coverage of every phase are unchanged
    assert sorted((t[0], t[1]) for t in _gemv_tasks(out)) == sorted((t[0], t[1]) for t in _gemv_tasks(b))


def test_batched_rebalance_keeps_the_16_row_groups(libamk):
    """A model of batch capacity 4 reads tile-major weights in 16-row groups: re-tiling for
    unequal rates moves boundaries in whole groups, stays valid, and still equalises the finish
    times to within that coarser alignment."""
    n_cu = 8
    blob = _tiny_blob(n_cu, batch=4)
    b = B.Blob(blob)
    rate = np.where(np.arange(n_cu) % 2 == 0, 0.02, 0.04)
    start = np.linspace(0.0, 1.0, n_cu)
    spread0 = _finish_spread(b, rate, start)
    out_blob = _lib.schedule_rebalance(blob, _trace(b, rate, start)[None], gain=1.0)
    out = B.Blob(out_blob)
    assert _lib.schedule_validate(out_blob)[0] == _lib.AMK_OK
    assert _lib.schedule_simulate(out_blob)[0] == _lib.AMK_OK
    moved = 0
    for (t0, t1) in zip(sorted(_gemv_tasks(b)), sorted(_gemv_tasks(out))):
        assert t1[4] % 16 == 0, t1
        moved += t0[4] != t1[4]
    assert moved > 0
    spread1 = _finish_spread(out, rate, start)
    assert spread1 < 0.5 * spread0 and spread1 <= 2 * 16 * 0.04 + 1e-9, (spread0, spread1)


def test_partial_gain_moves_part_of_the_way(libamk):
    blob = _tiny_blob()
    b = B.Blob(blob)
    rate = np.where(np.arange(8) < 4, 0.02, 0.04)
    start = np.zeros(8)
    full = B.Blob(_lib.schedule_rebalance(blob, _trace(b, rate, start)[None], gain=1.0))
    half = B.Blob(_lib.schedule_rebalance(blob, _trace(b, rate, start)[None], gain=0.5))
    rows = lambda x: {t[0]: t[5] - t[4] for t in _gemv_tasks(x)}
    r0, r1, rh = rows(b), rows(full), rows(half)
    for k in r0:
        lo, hi = sorted((r0[k], r1[k]))
        assert lo - 2 <= rh[k] <= hi + 2


def test_attention_waits_follow_the_qkv_tiles(libamk):
    """After re-tiling, every attention task waits on exactly the QKV tiles that cover its KV
    group's packed rows (the validator's race check relies on it; checked here directly)."""
    cfg = synth.get_config("tiny")
    blob = _tiny_blob()
    b = B.Blob(blob)
    rate = np.linspace(0.01, 0.05, 8)
    out = B.Blob(_lib.schedule_rebalance(blob, _trace(b, rate, np.zeros(8))[None], gain=1.0))
    grows = (cfg.n_heads // cfg.n_kv_heads + 2) * cfg.head_dim
    qkv = {}
    for tid, cu, mat, layer, a0, a1 in _gemv_tasks(out):
        if mat == B.M_QKV:
            qkv.setdefault(layer, []).append((tid, a0, a1))
    for v in out.per_cu:
        for t in v:
            if t["type"] != B.T_ATTN:
                continue
            g, l = int(t["a0"]), int(t["layer"])
            cover = [tid for tid, a0, a1 in qkv[l] if a0 < (g + 1) * grows and a1 > g * grows]
            assert (int(t["w0_lo"]), int(t["w0_hi"])) == (min(cover), max(cover) + 1)


def test_rebalance_rejects_bad_input(libamk):
    blob = _tiny_blob()
    b = B.Blob(blob)
    tr = _trace(b, np.full(8, 0.05))[None]
    for gain in (0.0, 1.5):
        with pytest.raises(_lib.AmkError) as e:
            _lib.schedule_rebalance(blob, tr, gain=gain)
        assert e.value.status == _lib.AMK_E_INVALID
    with pytest.raises(_lib.AmkError) as e:
        _lib.schedule_rebalance(blob[:64], tr, gain=0.5)
    # a trace without stamps leaves the tiles as they are
    out = _lib.schedule_rebalance(blob, np.zeros_like(tr), gain=1.0)
    assert {t[0]: t[4:] for t in _gemv_tasks(B.Blob(out))} == {t[0]: t[4:] for t in _gemv_tasks(b)}
