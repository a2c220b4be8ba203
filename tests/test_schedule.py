"""Schedule layer (host only): real lowerings validate and simulate clean; adversarial mutants
that the simulator finds unsafe are all rejected by the static validator (no false accepts)."""
import ctypes as C
import random

import numpy as np
import pytest

from persistent_decode_megakernel_amd import _lib, synth
from persistent_decode_megakernel_amd import blob as B

CONFIGS = ["tiny", "smollm2_135m", "tinyllama_1b", "llama2_7b", "llama2_7b_w8a16", "llama2_7b_w4a16"]


@pytest.mark.parametrize("name", CONFIGS)
def test_real_lowerings_validate(libamk, name):
    cfg = synth.get_config(name)
    c = _lib.make_config(cfg)
    for n_cu in (256, 304, 80):
        blob = _lib.schedule_build(c, cfg.batch, n_cu)
        st, rep = _lib.schedule_validate(blob)
        assert st == _lib.AMK_OK, rep
        b = B.Blob(blob)
        assert b.hdr.n_cu == n_cu and b.n_tasks == b.hdr.n_tasks
        ids = np.sort(b.all_tasks()["id"])
        assert np.array_equal(ids, np.arange(b.n_tasks))
        assert b.hdr.lds_bytes <= 160 * 1024


def test_search_parameters_and_predict(libamk):
    cfg = synth.get_config("llama2_7b")
    c = _lib.make_config(cfg)
    p = _lib.amk_sched_params(attn_blocks=4, placement=1, rotate=1, min_tile_kb=16, search=0)
    blob = _lib.schedule_build(c, 1, 256, p)
    b = B.Blob(blob)
    assert b.hdr.attn_blocks == 4 and b.hdr.placement == 1
    assert _lib.schedule_validate(blob)[0] == _lib.AMK_OK
    t1 = _lib.schedule_predict(blob, 2049)
    t2 = _lib.schedule_predict(blob, 4096)
    assert 0 < t1 < t2  # longer context, more KV bytes
    best = B.Blob(_lib.schedule_build(c, 1, 256))  # default: exhaustive search
    assert best.hdr.predicted_us <= _lib.schedule_predict(blob, c.max_seq) + 1e-6


def small_blobs():
    out = []
    for name, n_cu in (("tiny", 8), ("tiny", 13), ("smollm2_135m", 16)):
        cfg = synth.get_config(name)
        c = _lib.make_config(cfg)
        if name == "smollm2_135m":
            c.n_layers = 2
        for p in (None, _lib.amk_sched_params(placement=1, rotate=1, search=0)):
            out.append(_lib.schedule_build(c, 1, n_cu, p))
    return out


@pytest.mark.parametrize("idx", range(6))
def test_simulator_accepts_real_lowerings(libamk, idx):
    blob = small_blobs()[idx]
    st, rep = _lib.schedule_simulate(blob)
    assert st == _lib.AMK_OK, rep


def mutate(b: B.Blob, rng: random.Random) -> str:
    """Apply one random adversarial edit in place; return its kind."""
    cus = [c for c in range(len(b.per_cu)) if len(b.per_cu[c])]
    kind = rng.choice(["drop_wait", "shrink_wait", "shift_wait", "swap_same_cu", "move_cu",
                       "dup_rows", "gap_rows", "self_wait", "wait_later_same_cu", "widen_wait",
                       "reorder_cu", "bad_field", "attn_regroup", "attn_reblock",
                       "shrink_w1"])
    c = rng.choice(cus)
    v = b.per_cu[c]
    i = rng.randrange(len(v))
    t = v[i]
    if kind == "drop_wait":
        t["w0_lo"] = t["w0_hi"] = 0
    elif kind == "shrink_wait":
        if t["w0_hi"] > t["w0_lo"]:
            if rng.random() < 0.5:
                t["w0_hi"] -= 1
            else:
                t["w0_lo"] += 1
    elif kind == "shift_wait":
        d = rng.choice([-2, -1, 1, 2])
        t["w0_lo"] = max(0, int(t["w0_lo"]) + d)
        t["w0_hi"] = max(int(t["w0_lo"]), int(t["w0_hi"]) + d)
    elif kind == "widen_wait":
        t["w0_hi"] = min(b.hdr.n_tasks, int(t["w0_hi"]) + rng.randint(1, 50))
    elif kind == "swap_same_cu" and len(v) > 1:
        j = rng.randrange(len(v))
        v[[i, j]] = v[[j, i]]
    elif kind == "reorder_cu" and len(v) > 2:
        perm = list(range(len(v)))
        rng.shuffle(perm)
        b.per_cu[c] = v[perm]
    elif kind == "move_cu":
        c2 = rng.choice(range(len(b.per_cu)))
        task = v[i].copy()
        b.per_cu[c] = np.delete(v, i)
        pos = rng.randrange(len(b.per_cu[c2]) + 1)
        b.per_cu[c2] = np.insert(b.per_cu[c2], pos, task)
    elif kind == "dup_rows" and t["type"] == B.T_GEMV:
        t["a1"] = int(t["a1"]) + 2
    elif kind == "gap_rows" and t["type"] == B.T_GEMV and t["a1"] - t["a0"] > 2:
        t["a0"] = int(t["a0"]) + 2
    elif kind == "self_wait":
        t["w1_lo"], t["w1_hi"] = t["id"], t["id"] + 1
    elif kind == "wait_later_same_cu" and i + 1 < len(v):
        j = rng.randrange(i + 1, len(v))
        t["w1_lo"], t["w1_hi"] = v[j]["id"], v[j]["id"] + 1
    elif kind == "bad_field":
        t["a1"] = 10 ** 6
    elif kind == "shrink_w1":
        # a merger that skips one block of its group
        ms = [t2 for v2 in b.per_cu for t2 in v2 if t2["w1_hi"] > t2["w1_lo"] + 0 and t2["type"] == B.T_ATTN]
        if ms:
            t2 = rng.choice(ms)
            if rng.random() < 0.5:
                t2["w1_lo"] = int(t2["w1_lo"]) + 1
            else:
                t2["w1_hi"] = int(t2["w1_hi"]) - 1
    elif kind in ("attn_regroup", "attn_reblock"):
        # move a KV-block task to another group or block: two tasks write the same partials
        # and the group it left misses one (or its merger role no longer matches its block)
        attn = [(c2, j) for c2 in range(len(b.per_cu)) for j in range(len(b.per_cu[c2]))
                if b.per_cu[c2][j]["type"] == B.T_ATTN]
        c2, j = rng.choice(attn)
        t = b.per_cu[c2][j]
        field, top = ("a0", b.hdr.cfg.n_kv_heads) if kind == "attn_regroup" else ("a1", b.hdr.attn_blocks)
        if top > 1:
            t[field] = (int(t[field]) + rng.randrange(1, top)) % top
    return kind


def test_adversarial_corpus_zero_false_accepts(libamk):
    """Every mutant the dynamic simulator finds unsafe must be rejected by the validator; the
    validator may also reject mutants that happen to be safe (conservative), which is counted."""
    rng = random.Random(1234)
    bases = small_blobs()
    n_unsafe = n_safe = false_accepts = conservative = 0
    for k in range(600):
        b = B.Blob(rng.choice(bases))
        kinds = [mutate(b, rng) for _ in range(rng.choice([1, 1, 2]))]
        data = b.to_bytes()
        sv, rv = _lib.schedule_validate(data)
        ss, rs = _lib.schedule_simulate(data)
        if ss != _lib.AMK_OK:
            n_unsafe += 1
            if sv == _lib.AMK_OK:
                false_accepts += 1
                print("FALSE ACCEPT", kinds, rs)
        else:
            n_safe += 1
            if sv != _lib.AMK_OK:
                conservative += 1
    print(f"mutants: {n_unsafe} unsafe, {n_safe} safe, {conservative} safe-but-rejected")
    assert false_accepts == 0
    assert n_unsafe > 200


def test_truncated_and_corrupt_blobs_rejected(libamk):
    cfg = synth.get_config("tiny")
    blob = _lib.schedule_build(_lib.make_config(cfg), 1, 8)
    assert _lib.schedule_validate(blob[:100])[0] == _lib.AMK_E_SCHEDULE_REJECTED
    bad = bytearray(blob)
    bad[0] ^= 0xFF
    assert _lib.schedule_validate(bytes(bad))[0] == _lib.AMK_E_SCHEDULE_REJECTED
    b = B.Blob(blob)
    b.hdr.lds_bytes = 200 * 1024
    assert _lib.schedule_validate(b.to_bytes())[0] == _lib.AMK_E_SCHEDULE_REJECTED


@pytest.mark.parametrize("bad_offset", ["huge", "past_end", "non_monotone"])
def test_intermediate_offsets_checked_before_any_task_is_read(libamk, bad_offset):
    """Per-CU offsets of a blob whose first and last offsets are consistent but whose middle one
    points far past the task table: every parser entry rejects it without reading beyond the
    buffer (a parser that copied one CU's tasks before checking the next offset read past it)."""
    cfg = synth.get_config("tiny")
    blob = bytearray(_lib.schedule_build(_lib.make_config(cfg), 1, 8))
    h = B.BlobHeader.from_buffer_copy(bytes(blob[:C.sizeof(B.BlobHeader)]))
    off = np.frombuffer(bytes(blob), dtype="<u4", count=h.n_cu + 1, offset=h.offsets_off).copy()
    assert off[-1] == h.n_tasks and h.n_cu == 8
    off[1] = {"huge": 50_000_000, "past_end": h.n_tasks + 1000, "non_monotone": off[3] + 1}[bad_offset]
    if bad_offset == "non_monotone":
        off[2] = off[1] - 2
    blob[h.offsets_off:h.offsets_off + 4 * (h.n_cu + 1)] = off.astype("<u4").tobytes()
    data = bytes(blob)
    st, rep = _lib.schedule_validate(data)
    assert st == _lib.AMK_E_SCHEDULE_REJECTED and "offsets" in rep, rep
    assert _lib.schedule_simulate(data)[0] == _lib.AMK_E_SCHEDULE_REJECTED


def FOUR_BLOCKS():
    return _lib.amk_sched_params(attn_blocks=4, search=0)


def _attn(b: B.Blob, layer: int):
    """[(cu, index)] of the layer's O tiles; sorted ids of its mergers and of its other blocks."""
    o = [(c, j) for c in range(len(b.per_cu)) for j in range(len(b.per_cu[c]))
         if b.per_cu[c][j]["type"] == B.T_GEMV and b.per_cu[c][j]["mat"] == B.M_O
         and b.per_cu[c][j]["layer"] == layer]
    attn = [t for v in b.per_cu for t in v if t["type"] == B.T_ATTN and t["layer"] == layer]
    mergers = sorted(int(t["id"]) for t in attn if t["aux1"])
    others = sorted(int(t["id"]) for t in attn if not t["aux1"])
    return o, mergers, others


def _ranges(b: B.Blob, cfg):
    """head ranges per KV group of a schedule's attention tasks"""
    hp = {int(t["aux3"]) for v in b.per_cu for t in v if t["type"] == B.T_ATTN}
    assert len(hp) == 1
    return (cfg.n_heads // cfg.n_kv_heads) // hp.pop()


@pytest.mark.parametrize("drop", ["first", "last"])
def test_o_tile_must_wait_for_every_merger(libamk, drop):
    """The last block of each (KV group, query-head range) merges the range's partials into the
    attention output, so an O-projection tile that skips any one merger may read an unmerged
    output: the validator rejects it and the delayed-CU simulation shows the stale read."""
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg), 1, 8, FOUR_BLOCKS()))
    o, mergers, others = _attn(b, 1)
    assert len(mergers) == cfg.n_kv_heads * _ranges(b, cfg) and mergers[0] > max(others)
    dropped = mergers[0] if drop == "first" else mergers[-1]
    cu_of = {int(t["id"]): c for c in range(len(b.per_cu)) for t in b.per_cu[c]}
    c, j = next((c, j) for c, j in o if c != cu_of[dropped])
    t = b.per_cu[c][j]
    assert (int(t["w0_lo"]), int(t["w0_hi"])) == (mergers[0], mergers[-1] + 1)
    if drop == "first":
        t["w0_lo"] = mergers[0] + 1
    else:
        t["w0_hi"] = mergers[-1]
    data = b.to_bytes()
    st, rep = _lib.schedule_validate(data)
    assert st == _lib.AMK_E_SCHEDULE_REJECTED and "race" in rep, rep
    assert _lib.schedule_simulate(data)[0] != _lib.AMK_OK


@pytest.mark.parametrize("max_batch", [1, 2])
def test_merger_must_wait_for_every_block_of_its_group(libamk, max_batch):
    """A merger that skips its range's last sibling. Batched (flag waits): the race is real,
    the validator reports it and the delayed-CU simulation shows the stale read. Batch 1: the
    declared waits no longer equal the writers of the merger's tagged inputs, rejected."""
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg, max_batch=max_batch), 1, 8, FOUR_BLOCKS()))
    o, mergers, others = _attn(b, 0)
    t = next(t for v in b.per_cu for t in v if int(t["id"]) == mergers[0])
    assert int(t["w1_hi"]) - int(t["w1_lo"]) == b.hdr.attn_blocks - 1 > 0
    t["w1_hi"] = int(t["w1_hi"]) - 1
    data = b.to_bytes()
    st, rep = _lib.schedule_validate(data)
    assert st == _lib.AMK_E_SCHEDULE_REJECTED, rep
    if max_batch == 1:
        assert "writers" in rep or "race" in rep, rep
    else:
        assert "race" in rep, rep
        assert _lib.schedule_simulate(data)[0] != _lib.AMK_OK


def test_merger_must_be_the_groups_last_block(libamk):
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg), 1, 8, FOUR_BLOCKS()))
    for v in b.per_cu:
        for t in v:
            if t["type"] == B.T_ATTN and t["layer"] == 0 and t["a0"] == 0 and t["a1"] == 0:
                t["aux1"] = 1
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_E_SCHEDULE_REJECTED and "merger" in rep, rep


def _tasks_by(b: B.Blob, typ, mat=None, layer=None):
    return sorted(int(t["id"]) for v in b.per_cu for t in v
                  if t["type"] == typ and (mat is None or t["mat"] == mat)
                  and (layer is None or t["layer"] == layer))


def _find(b: B.Blob, tid: int):
    return next(t for v in b.per_cu for t in v if int(t["id"]) == tid)


@pytest.mark.parametrize("max_batch", [1, 2])
def test_tagged_tile_waits_must_equal_its_input_writers(libamk, max_batch):
    """Batch-1 instances: a gate/up tile waits by reloading its tagged input, so a declared wait
    on anything other than that input's writers (here also an attention block, harmless as a flag
    wait) would be a dependency the kernel never enforces: rejected. The batched instance waits on
    flags, where the extra wait is merely redundant: accepted."""
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg, max_batch=max_batch), 1, 8))
    gu = _tasks_by(b, B.T_GEMV, B.M_GU, 1)
    attn = _tasks_by(b, B.T_ATTN, None, 1)
    t = _find(b, gu[0])
    assert int(t["w1_lo"]) == int(t["w1_hi"])
    t["w1_lo"], t["w1_hi"] = attn[0], attn[0] + 1
    st, rep = _lib.schedule_validate(b.to_bytes())
    if max_batch == 1:
        assert st == _lib.AMK_E_SCHEDULE_REJECTED and "tagged" in rep, rep
    else:
        assert st == _lib.AMK_OK, rep


@pytest.mark.parametrize("max_batch", [1, 2])
def test_flag_wait_on_a_tile_that_stores_no_flag(libamk, max_batch):
    """Batch-1 O, gate/up and down tiles publish tagged data and no flag: a task that waits on
    flags (here the argmax, also on a down tile) would wait forever. Batched tiles store flags."""
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg, max_batch=max_batch), 1, 8))
    dn = _tasks_by(b, B.T_GEMV, B.M_D, cfg.n_layers - 1)
    t = _find(b, _tasks_by(b, B.T_ARGMAX)[0])
    assert int(t["w1_lo"]) == int(t["w1_hi"])
    t["w1_lo"], t["w1_hi"] = dn[0], dn[0] + 1
    st, rep = _lib.schedule_validate(b.to_bytes())
    if max_batch == 1:
        assert st == _lib.AMK_E_SCHEDULE_REJECTED and "stores none" in rep, rep
    else:
        assert st == _lib.AMK_OK, rep


def test_tagged_waits_of_real_lowerings_are_their_input_writers(libamk):
    """Dropping one writer from a tagged tile's waits (a shrunk range) is rejected even where the
    tile's CU order happens to cover it."""
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg), 1, 8))
    d = _tasks_by(b, B.T_GEMV, B.M_D, 0)
    gu = _tasks_by(b, B.T_GEMV, B.M_GU, 0)
    t = _find(b, d[0])
    assert (int(t["w0_lo"]), int(t["w0_hi"])) == (gu[0], gu[-1] + 1)
    t["w0_hi"] = gu[-1]
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_E_SCHEDULE_REJECTED, rep


def test_schedule_without_an_argmax_is_rejected(libamk):
    """Several steps run in one launch: a step's first tiles wait on the previous step's argmax,
    which must therefore exist and follow every task of the step. Without one the validator
    rejects the schedule before looking at output coverage."""
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg), 1, 8))
    am = _tasks_by(b, B.T_ARGMAX)
    assert am == [b.n_tasks - 1]
    for c, v in enumerate(b.per_cu):
        b.per_cu[c] = v[v["type"] != B.T_ARGMAX]
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_E_SCHEDULE_REJECTED and "argmax" in rep, rep


def test_int4_weight_bytes_and_config_checks(libamk):
    """W4A16: the schedule's byte model counts half a byte per weight plus one fp32 scale per row
    and group; configurations the int4 kernels cannot take are refused by the builder."""
    cfg = synth.get_config("llama2_7b_w4a16")
    c4 = _lib.make_config(cfg)
    c8 = _lib.make_config(synth.get_config("llama2_7b_w8a16"))
    p4 = _lib.schedule_predict(_lib.schedule_build(c4, 1, 256), 4096)
    p8 = _lib.schedule_predict(_lib.schedule_build(c8, 1, 256), 4096)
    assert p4 < p8
    for bad in (dict(group=48), dict(group=16), dict(ffn=11008 + 32), dict(hidden=64, n_heads=1,
                                                                            head_dim=64)):
        with pytest.raises(_lib.AmkError) as e:
            _lib.schedule_build(_lib.make_config(cfg.replace(**bad)), 1, 256)
        assert e.value.status == _lib.AMK_E_INVALID
    # a group size on a non-int4 model is refused too
    c = _lib.make_config(synth.get_config("llama2_7b"))
    c.group_size = 128
    with pytest.raises(_lib.AmkError):
        _lib.schedule_build(c, 1, 256)


def _gemv_phases(b: B.Blob):
    ph = {}
    for v in b.per_cu:
        for t in v:
            if t["type"] == B.T_GEMV:
                ph.setdefault((int(t["mat"]), int(t["layer"])), []).append(t)
    for k in ph:
        ph[k].sort(key=lambda t: int(t["a0"]))
    return ph


@pytest.mark.parametrize("name,max_batch", [("llama2_7b", 8), ("llama2_7b", 16), ("tiny", 3),
                                            ("smollm2_135m", 4), ("llama2_7b_w4a16", 2)])
def test_batched_tiles_follow_the_16_row_weight_groups(libamk, name, max_batch):
    """A model of batch capacity above 1 stores its weights tile-major in 16-row groups, so each
    GEMV tile of its schedules starts on a group boundary (the last ends at the matrix's rows) and
    the validator rejects a boundary moved off one, even by a whole row pair."""
    cfg = synth.get_config(name)
    c = _lib.make_config(cfg, max_batch=max_batch)
    for batch in sorted({1, max_batch}):
        b = B.Blob(_lib.schedule_build(c, batch, 256))
        assert _lib.schedule_validate(b.to_bytes())[0] == _lib.AMK_OK
        for (mat, layer), v in _gemv_phases(b).items():
            assert int(v[0]["a0"]) == 0
            for t0, t1 in zip(v, v[1:]):
                assert int(t0["a1"]) == int(t1["a0"]) and int(t1["a0"]) % 16 == 0, (mat, layer)
    # shift one gate/up boundary by a row pair: pair-aligned, complete, but off the groups (the
    # tile that grows stays within the tallest tile, which the LDS size covers; 13 CUs make the
    # tiles uneven)
    b = B.Blob(_lib.schedule_build(c, max_batch, 13))
    assert _lib.schedule_validate(b.to_bytes())[0] == _lib.AMK_OK
    ph = _gemv_phases(b)
    tallest = max(int(t["a1"]) - int(t["a0"]) for v in ph.values() for t in v)
    v = ph[(B.M_GU, 0)]
    i = next(i for i in range(len(v) - 1) if int(v[i]["a1"]) - int(v[i]["a0"]) > 2
             and int(v[i + 1]["a1"]) - int(v[i + 1]["a0"]) + 2 <= tallest)
    v[i]["a1"] = int(v[i]["a1"]) - 2
    v[i + 1]["a0"] = int(v[i + 1]["a0"]) - 2
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_E_SCHEDULE_REJECTED and "16-row" in rep, rep


def test_batch1_tiles_keep_row_pairs_only(libamk):
    """Batch-1 models keep row-major weights: tiles need only whole RoPE / SwiGLU pairs, and a
    boundary moved by a pair is still valid."""
    cfg = synth.get_config("tiny")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg), 1, 8))
    v = _gemv_phases(b)[(B.M_GU, 0)]
    i = next(i for i in range(len(v) - 1) if int(v[i]["a1"]) - int(v[i]["a0"]) > 2)
    v[i]["a1"] = int(v[i]["a1"]) - 2
    v[i + 1]["a0"] = int(v[i + 1]["a0"]) - 2
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_OK, rep
    v[i]["a1"] = int(v[i]["a1"]) - 1
    v[i + 1]["a0"] = int(v[i + 1]["a0"]) - 1
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_E_SCHEDULE_REJECTED and "row pair" in rep, rep


@pytest.mark.parametrize("name,hp,ranges", [("tiny", 0, None), ("tiny", 2, 1), ("tiny", 1, 2),
                                            ("tiny", 3, 1), ("smollm2_135m", 0, None),
                                            ("tinyllama_1b", 0, None), ("tinyllama_1b", 2, 4),
                                            ("tinyllama_1b", 8, 1), ("llama2_7b", 0, 1)])
def test_query_head_ranges(libamk, name, hp, ranges):
    """Attention tasks cover a range of their group's query heads (aux2 = first head, aux3 =
    heads). Batch 1 splits a group so that up to two attention tasks run per CU unless told
    otherwise; a heads_per_task that does not divide the group's heads keeps whole groups. Each
    (group, range) has its own blocks and merger, every block waits on the QKV tiles of its whole
    group, the O tiles wait on all mergers; the schedule validates and simulates clean."""
    cfg = synth.get_config(name)
    qpg = cfg.n_heads // cfg.n_kv_heads
    p = _lib.amk_sched_params(search=0, heads_per_task=hp)
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg, max_seq=cfg.prefill + 8), 1, 256, p))
    data = b.to_bytes()
    assert _lib.schedule_validate(data)[0] == _lib.AMK_OK
    assert _lib.schedule_simulate(data)[0] == _lib.AMK_OK
    nblk = int(b.hdr.attn_blocks)
    if ranges is None:  # auto: the most ranges (a divisor of the group's heads) within 2 tasks per CU
        ranges = max(r for r in range(1, qpg + 1) if qpg % r == 0 and cfg.n_kv_heads * r * nblk <= 512)
    assert _ranges(b, cfg) == ranges
    attn = [t for v in b.per_cu for t in v if t["type"] == B.T_ATTN and t["layer"] == 0]
    assert len(attn) == cfg.n_kv_heads * ranges * nblk
    heads = {}
    for t in attn:
        heads.setdefault((int(t["a0"]), int(t["a1"])), []).append((int(t["aux2"]), int(t["aux3"])))
    for key, rs in heads.items():  # the ranges of a (group, block) tile the group's heads
        covered = sorted(h for h0, n in rs for h in range(h0, h0 + n))
        assert covered == list(range(qpg)), (key, rs)
    mergers = [t for t in attn if t["aux1"]]
    assert len(mergers) == cfg.n_kv_heads * ranges
    assert all(int(t["a1"]) == nblk - 1 for t in mergers)


def test_head_range_outside_the_group_is_rejected(libamk):
    cfg = synth.get_config("tinyllama_1b")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg, max_seq=cfg.prefill + 8), 1, 256,
                                   _lib.amk_sched_params(search=0)))
    t = next(t for v in b.per_cu for t in v if t["type"] == B.T_ATTN)
    t["aux2"] = 8 - int(t["aux3"]) + 1
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_E_SCHEDULE_REJECTED and "head range" in rep, rep


def test_overlapping_head_ranges_are_rejected(libamk):
    """Two blocks writing the same head's partial: the single-writer rule catches it."""
    cfg = synth.get_config("tinyllama_1b")
    b = B.Blob(_lib.schedule_build(_lib.make_config(cfg, max_seq=cfg.prefill + 8), 1, 256,
                                   _lib.amk_sched_params(search=0)))
    t = next(t for v in b.per_cu for t in v if t["type"] == B.T_ATTN and int(t["aux2"]) > 0
             and not t["aux1"])
    t["aux2"] = int(t["aux2"]) - 1
    st, rep = _lib.schedule_validate(b.to_bytes())
    assert st == _lib.AMK_E_SCHEDULE_REJECTED, rep
