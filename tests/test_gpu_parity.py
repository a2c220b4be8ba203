"""HIP path vs the CPU oracle, element by element, through the C ABI (GPU only)."""
import numpy as np
import pytest
import torch

from persistent_decode_megakernel_amd import synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import assert_parity, log, teacher_forced

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_tiny_teacher_forced(path):
    """Tiny config: 32 prompt ids fed one by one, then 16 greedy steps (47 calls), p = 0..46."""
    rep = teacher_forced(synth.get_config("tiny"), path)
    log(f"tiny/{path}: {rep}")
    assert rep.steps == 47
    assert_parity(rep)


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_tiny_random_gains(path):
    """Norm gains 1 + N(0, 0.02): a kernel that ignored a gain would fail here."""
    rep = teacher_forced(synth.get_config("tiny"), path, seed=1, n_calls=12, random_gains=True)
    assert_parity(rep)


def test_tiny_free_running_matches_oracle_until_low_margin():
    import oracle
    cfg = synth.get_config("tiny")
    w = synth.make_weights(cfg, 2)
    params, wn = synth.oracle_inputs(w)
    dec = oracle.Decoder(params, wn)
    kv_np = np.zeros((cfg.n_layers, 2, 1, cfg.n_kv_heads, cfg.max_seq, cfg.head_dim), np.uint16)
    toks = synth.make_tokens(cfg, 2).numpy()[0]
    model = Model(cfg, w)
    kv = model.kv()
    d_tok = torch.tensor([int(toks[0])], dtype=torch.int32, device="cuda")
    gpu_ids, ora_ids, margins = [], [], []
    tok = int(toks[0])
    for i in range(cfg.n_calls):
        lo = dec.step(kv_np, np.array([tok]), i)
        nxt = model.step(kv, d_tok, i, next_out=None)
        ora = int(oracle.argmax_lowest(lo)[0])
        margins.append(float(oracle.top2_margin(lo)[0]))
        if i + 1 < cfg.prompt:
            tok = int(toks[i + 1])
            d_tok = torch.tensor([tok], dtype=torch.int32, device="cuda")
        else:
            gpu_ids.append(int(nxt.item()))
            ora_ids.append(ora)
            tok = ora
            d_tok = nxt  # on-device greedy chaining
        model.sync()
    gen_margins = margins[cfg.prompt - 1:]
    for i, (g, o) in enumerate(zip(gpu_ids, ora_ids)):
        if gen_margins[i] <= 0.05:
            break
        assert g == o, f"generated token {i}: gpu {g} oracle {o}"
    kv.close()
    model.close()


def test_smollm2_135m_teacher_forced():
    rep = teacher_forced(synth.get_config("smollm2_135m"), "megakernel", n_calls=8)
    log(f"135m: {rep}")
    assert_parity(rep)


def test_tinyllama_1b_teacher_forced():
    rep = teacher_forced(synth.get_config("tinyllama_1b"), "megakernel", n_calls=3,
                         oracle_dtype=np.float32)
    log(f"1.1b: {rep}")
    assert_parity(rep)


@pytest.mark.parametrize("pos", [0, 1, 5])
def test_first_positions_and_empty_kv_blocks(pos):
    """ctx = pos + 1 smaller than the number of KV blocks: most blocks are empty."""
    cfg = synth.get_config("smollm2_135m").replace(prefill=pos)
    rep = teacher_forced(cfg, "megakernel", n_calls=2, first_pos=pos)
    assert_parity(rep)


def test_last_position():
    cfg = synth.get_config("tiny")
    rep = teacher_forced(cfg.replace(prefill=40, prompt=0, steps=7), "megakernel", n_calls=7)
    assert_parity(rep)


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_tiny_int8_w8a16(path):
    """W8A16: int8 layer matrices and LM head with per-row fp32 scales."""
    cfg = synth.get_config("tiny").replace(wtype="int8")
    rep = teacher_forced(cfg, path, seed=3, n_calls=20)
    log(f"tiny int8/{path}: {rep}")
    assert_parity(rep)


def test_int8_hidden_4096_two_rows_per_chunk():
    """W8A16 with hidden 4096 (32 heads of 128, 8 KV heads): batch-1 int8 rows of K = 4096 (QKV, O,
    gate/up, LM head) run two rows per weight chunk, the down rows (K = 688) one ragged row per
    chunk; the input goes to the integer dot products as digits. Random norm gains widen the
    input's range."""
    cfg = synth.get_config("tiny").replace(wtype="int8", hidden=4096, n_heads=32, n_kv_heads=8,
                                           head_dim=128)
    rep = teacher_forced(cfg, "megakernel", seed=6, n_calls=12, random_gains=True)
    log(f"int8 hidden 4096: {rep}")
    assert_parity(rep)


# int4 groups must divide the FFN: the tiny shape with FFN 768 and groups of 128
TINY_INT4 = dict(wtype="int4", ffn=768, group=128)


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_tiny_int4_w4a16(path):
    """W4A16: packed int4 layer matrices and LM head with one fp32 scale per row and group."""
    cfg = synth.get_config("tiny").replace(**TINY_INT4)
    rep = teacher_forced(cfg, path, seed=3, n_calls=20)
    log(f"tiny int4/{path}: {rep}")
    assert_parity(rep)


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_tiny_int4_batch3(path):
    """Batched W4A16 on the matrix cores: nibbles as exact bf16 (q + 136), a correction product
    for the offset, each k step scaled by its group's scale."""
    cfg = synth.get_config("tiny").replace(batch=3, **TINY_INT4)
    rep = teacher_forced(cfg, path, seed=4, n_calls=12)
    assert rep.tokens_checked > 0
    assert_parity(rep)


def test_int4_hidden_4096_four_rows_per_chunk():
    """W4A16 with hidden 4096 and groups of 64: batch-1 int4 rows of K = 4096 run four rows per
    weight chunk, the down rows (K = 768) one ragged row per chunk."""
    cfg = synth.get_config("tiny").replace(wtype="int4", hidden=4096, n_heads=32, n_kv_heads=8,
                                           head_dim=128, ffn=768, group=64)
    rep = teacher_forced(cfg, "megakernel", seed=7, n_calls=12, random_gains=True)
    log(f"int4 hidden 4096: {rep}")
    assert_parity(rep)


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_tiny_batch3(path):
    """Three independent sequences sharing the weights and the position."""
    cfg = synth.get_config("tiny").replace(batch=3)
    rep = teacher_forced(cfg, path, seed=4, n_calls=12)
    assert rep.tokens_checked > 0
    assert_parity(rep)


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_batch3_tiles_off_the_grid(path):
    """A batched model's tile-major weights end in zero-padded tiles: 4100 vocabulary rows
    leave the LM head a last 16-row group of 4 rows, and a 696-wide FFN gives the down projection
    21.75 steps of 32 inputs."""
    cfg = synth.get_config("tiny").replace(batch=3, ffn=696, vocab=4100)
    rep = teacher_forced(cfg, path, seed=12, n_calls=8)
    assert rep.tokens_checked > 0
    assert_parity(rep)


@pytest.mark.parametrize("path", ["megakernel", "unfused"])
def test_tiny_batch16(path):
    """Sixteen sequences: the matrix cores take one column per sequence and multiply the two bf16
    halves of the input by two instructions."""
    cfg = synth.get_config("tiny").replace(batch=16)
    rep = teacher_forced(cfg, path, seed=8, n_calls=6)
    assert rep.tokens_checked > 0
    assert_parity(rep)


def test_smollm2_135m_batch2_prefill():
    cfg = synth.get_config("smollm2_135m").replace(batch=2)
    rep = teacher_forced(cfg, "megakernel", seed=5, n_calls=3)
    assert_parity(rep)


@pytest.mark.parametrize("name", ["llama2_7b", "llama2_7b_w8a16", "llama2_7b_w4a16", "llama2_7b_b8",
                                  "llama2_7b_b16"])
def test_full_size_first_steps(name):
    """Full 7B shapes in the launch configuration the bench times (one cooperative launch per
    step on every CU), checked against the oracle on every logit for the first two steps."""
    cfg = synth.get_config(name)
    rep = teacher_forced(cfg, "megakernel", n_calls=2, oracle_dtype=np.float32)
    log(f"{name}: {rep}")
    assert_parity(rep)
