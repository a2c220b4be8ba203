"""The unfused ablation launched as hipGraph replays (one captured graph per position, since the
position is a launch argument): every replay reproduces the eager launches' logits bit for bit,
with eager work and host synchronisations between replays. GPU only."""
import numpy as np
import pytest
import torch

from persistent_decode_megakernel_amd import synth
from persistent_decode_megakernel_amd.model import Model

from gpu_helpers import log

pytestmark = pytest.mark.gpu


def test_unfused_graph_replays_match_eager():
    cfg = synth.get_config("tiny")
    w = synth.make_weights(cfg, 7, threads=16)
    n = 6
    max_seq = cfg.max_seq
    model = Model(cfg, w, path="unfused", max_seq=max_seq)
    kv = model.kv(cfg.batch, max_seq)
    toks = synth.make_tokens(cfg, 7).numpy()[0, :n].astype(np.int32)
    tok = torch.empty(cfg.batch, dtype=torch.int32, device="cuda")
    nxt = torch.empty_like(tok)
    logits = torch.empty((cfg.batch, cfg.vocab), dtype=torch.float32, device="cuda")

    eager = []
    kv.tensor.zero_()
    for p in range(n):
        tok.fill_(int(toks[p]))
        model.step(kv, tok, p, logits, next_out=nxt)
        model.sync()
        eager.append((logits.cpu().numpy().copy(), int(nxt.item())))

    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    graphs = []
    with torch.cuda.stream(cap):
        for p in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                model.step(kv, tok, p, logits, next_out=nxt)
            graphs.append(g)
    stream.wait_stream(cap)
    torch.cuda.synchronize()

    for rep in range(3):
        kv.tensor.zero_()  # eager work between replays
        torch.cuda.synchronize()
        for p in range(n):
            tok.fill_(int(toks[p]))
            graphs[p].replay()
            torch.cuda.synchronize()
            lg = logits.cpu().numpy()
            assert np.array_equal(lg, eager[p][0]), f"replay {rep} position {p}: logits differ"
            assert int(nxt.item()) == eager[p][1]
        log(f"  graph replay pass {rep}: {n} positions bit-identical to eager launches")
    del graphs
    kv.close()
    model.close()
