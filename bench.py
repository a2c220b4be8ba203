"""Decode throughput of the persistent megakernel on one MI355X.

A step is one full decode step (embedding through greedy argmax) of the workload's model on a
batch of synthetic input, greedy ids chained on the device. Prints ONE JSON line with
tokens/s, the achieved HBM rate of the megakernel against MI355X's 8 TB/s, the unfused
ablation measured in the same run, and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 64] [--warmup 3] [--workload llama2_7b]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kv_bytes_step(cfg, ctx):
    return cfg.batch * cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * 2 * ctx


def time_path(cfg, weights, kv_host, path, steps, warmup, graph=False):
    """Returns (ms per step from events around the whole timed region, per-launch durations ms,
    model info, final token ids). graph=True: each timed step is one hipGraph replay of the step's
    launches (captured beforehand, one graph per position, since the position is a launch argument)."""
    import torch
    from persistent_decode_megakernel_amd import synth
    from persistent_decode_megakernel_amd.model import Model

    max_seq = cfg.prefill + max(steps, warmup) + 1
    t0 = time.time()
    model = Model(cfg, weights, path=path, max_seq=max_seq)
    info = model.info()
    kv = model.kv(cfg.batch, max_seq)
    kv.tensor.copy_(kv_host[..., :max_seq, :].to(kv.tensor.device))
    log(f"[bench] {path}{' (hipGraph)' if graph else ''}: model ready in {time.time() - t0:.1f}s "
        f"({info.n_tasks} tasks on {info.n_cu} CUs, {info.launches_per_step} launches/step)")
    first = synth.make_tokens(cfg, 0)[:, 0].to(torch.int32).cuda()
    tok = torch.empty_like(first)
    stream = torch.cuda.current_stream()
    graphs = []
    if graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for i in range(steps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    model.step(kv, tok, cfg.prefill + i, next_out=tok)
                graphs.append(g)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
    # warmup (positions P .. P+W-1), then the timed region restarts at P
    tok.copy_(first)
    for i in range(warmup):
        model.step(kv, tok, cfg.prefill + i, next_out=tok)
    model.sync()
    torch.cuda.synchronize()
    tok.copy_(first)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        if graph:
            graphs[i].replay()
        else:
            model.step(kv, tok, cfg.prefill + i, next_out=tok)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    model.sync()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    total = ev[0].elapsed_time(ev[steps])
    ids = tok.cpu().tolist()
    del graphs
    kv.close()
    model.close()
    del kv, model
    torch.cuda.empty_cache()
    return total / steps, per, info, ids


def time_multistep(cfg, weights, kv_host, steps, warmup):
    """The same positions as time_path's megakernel run, decoded as ONE launch of `steps` greedy
    steps (amk_decode_steps: each step's first tiles wait on the previous step's argmax inside the
    kernel). Returns (ms per step, final token ids)."""
    import torch
    from persistent_decode_megakernel_amd import synth
    from persistent_decode_megakernel_amd.model import Model

    max_seq = cfg.prefill + max(steps, warmup) + 1
    model = Model(cfg, weights, path="megakernel", max_seq=max_seq)
    kv = model.kv(cfg.batch, max_seq)
    kv.tensor.copy_(kv_host[..., :max_seq, :].to(kv.tensor.device))
    first = synth.make_tokens(cfg, 0)[:, 0].to(torch.int32).cuda()
    out = torch.empty((max(steps, warmup), cfg.batch), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    if warmup:
        model.steps(kv, first, cfg.prefill, warmup, out=out[:warmup])
    model.sync()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    model.steps(kv, first, cfg.prefill, steps, out=out[:steps])
    ev[1].record(stream)
    torch.cuda.synchronize()
    model.sync()
    ms = ev[0].elapsed_time(ev[1]) / steps
    ids = out[steps - 1].cpu().tolist()
    kv.close()
    model.close()
    del kv, model
    torch.cuda.empty_cache()
    return ms, ids


def time_prompt_scenario(cfg, weights, n_in=64, n_out=12, reps=3):
    """The pages' fixed short-sequence scenario (input 64 tokens, output 12; Ada-MK summary,
    "Experimental Results"), from an empty cache. Hybrid: the prompt through amk_prefill (up to 16
    tokens per matrix-core pass), then the 12 greedy steps as one megakernel launch. Decode only:
    the 64 prompt tokens fed as 64 single megakernel steps, then the same 12 steps. Returns ms of
    each (best of `reps`) and whether both produced the same 12 tokens."""
    import numpy as np
    import torch
    from persistent_decode_megakernel_amd.model import Model

    cfg1 = cfg.replace(batch=1)
    max_seq = n_in + n_out + 1
    model = Model(cfg1, weights, path="megakernel", max_seq=max_seq)
    prompt = torch.from_numpy(
        np.random.default_rng(64).integers(0, cfg.vocab, n_in).astype(np.int32)).cuda()
    stream = torch.cuda.current_stream()
    best = {"hybrid": 1e30, "decode_only": 1e30}
    outs = {}
    for _ in range(reps):
        for mode in ("hybrid", "decode_only"):
            kv = model.kv(1, max_seq)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            if mode == "hybrid":
                nxt = model.prefill(kv, prompt, 0)
            else:
                nxt = torch.empty(1, dtype=torch.int32, device="cuda")
                for i in range(n_in):
                    model.step(kv, prompt[i:i + 1], i, next_out=nxt)
            out = model.steps(kv, nxt, n_in, n_out)
            ev[1].record(stream)
            torch.cuda.synchronize()
            model.sync()
            best[mode] = min(best[mode], ev[0].elapsed_time(ev[1]))
            outs[mode] = out.cpu().numpy().ravel().tolist()
            kv.close()
    model.close()
    torch.cuda.empty_cache()
    return {"input_tokens": n_in, "output_tokens": n_out,
            "hybrid_ms": round(best["hybrid"], 3), "decode_only_ms": round(best["decode_only"], 3),
            "hybrid_speedup": round(best["decode_only"] / best["hybrid"], 3),
            "same_output_tokens": outs["hybrid"] == outs["decode_only"]}


def profiled_traffic(cfg, kernel_name):
    """Per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from the committed
    rocprofv3 summary of this workload, or None when the kernel sources changed since."""
    from persistent_decode_megakernel_amd import profile_summary
    path = os.path.join(ROOT, "profiles", f"megakernel_{cfg.name}_b{cfg.batch}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel_name or rec.get("source_hash") != profile_summary.source_hash():
        return None
    return float(rec["traffic_bytes_per_launch"])


def cpu_baseline(cfg, weights, kv_host, sample_steps):
    """The oracle (float64 numpy, as it stands) on a bounded sample of the same workload: the first
    `sample_steps` decode steps of the full model from the same prefilled cache and first token."""
    import numpy as np
    import oracle
    from persistent_decode_megakernel_amd import synth

    params, wn = synth.oracle_inputs(weights)
    pos = cfg.prefill
    kv = synth.bf16_to_numpy_bits(kv_host[..., :pos + sample_steps, :]).copy()
    tok = synth.make_tokens(cfg, 0)[:, 0].numpy()
    dec = oracle.Decoder(params, wn, cache_bytes=0)
    t = time.perf_counter()
    for i in range(sample_steps):
        logits = dec.step(kv, tok, pos + i)
        tok = oracle.argmax_lowest(logits)
    t_step = (time.perf_counter() - t) / sample_steps
    cores = len(os.sched_getaffinity(0))
    threads = cores
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = int(info[0].get("num_threads", cores))
    except Exception:
        pass
    return {
        "value": round(cfg.batch / t_step, 4),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{sample_steps} greedy decode steps of the full {cfg.name} model at positions "
                   f"{pos}..{pos + sample_steps - 1} ({t_step:.1f} s per step), float64 numpy "
                   f"matrix-vector products, weights converted per matrix per step; host has "
                   f"{cores} cores"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama2_7b")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-multistep", action="store_true")
    ap.add_argument("--no-scenario", action="store_true")
    ap.add_argument("--batch", type=int, default=0,
                    help="override the workload's batch (sequences per step, 1..16)")
    ap.add_argument("--cpu-sample-steps", type=int, default=2)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB first (a kernel of "
                         "known traffic for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the decode "
              "step runs on a single MI355X; multi-GPU sharding is a design note, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from persistent_decode_megakernel_amd import _lib, synth

    _lib.load()
    torch.cuda.set_device(0)
    cfg = synth.get_config(args.workload)
    if args.batch:
        cfg = cfg.replace(batch=args.batch)
    steps, warmup = args.steps, args.warmup
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n} bytes read, {n} bytes written")
        del src, dst
    t0 = time.time()
    weights = synth.make_weights(cfg, 0, threads=16)
    max_seq = cfg.prefill + max(steps, warmup) + 1
    kv_host = synth.make_kv(cfg, max_seq, 0, threads=16)
    log(f"[bench] synthetic {cfg.name} generated in {time.time() - t0:.1f}s")

    ms, per, info, ids = time_path(cfg, weights, kv_host, "megakernel", steps, warmup)
    hd_q = 1 if cfg.n_heads // cfg.n_kv_heads <= 1 else (2 if cfg.n_heads // cfg.n_kv_heads <= 2 else 4)
    wt = {"bf16": 0, "int8": 1, "int4": 2}[cfg.wtype]
    kname = (f"amk_megakernel_w{wt}_h{cfg.head_dim}_q{hd_q}"
             + ("_b" if cfg.batch > 1 else ""))
    traffic_bytes = profiled_traffic(cfg, kname)
    weight_bytes = info.weight_bytes + 2 * cfg.hidden * cfg.batch  # + embedding rows
    ctxs = [cfg.prefill + i + 1 for i in range(steps)]
    step_bytes = [weight_bytes + kv_bytes_step(cfg, c) for c in ctxs]
    avg_bytes = sum(step_bytes) / steps
    avg_launch_ms = sum(per) / steps  # one launch per step
    achieved = avg_bytes / (avg_launch_ms * 1e-3) / 1e9
    value = cfg.batch * steps / (ms * steps * 1e-3)
    out = {
        "metric": "decode tokens/s at batch 1 + achieved HBM GB/s as % of 8 TB/s peak",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.wtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.n_layers} layers, hidden {cfg.hidden}, "
                        f"{cfg.n_heads}/{cfg.n_kv_heads} heads, head_dim {cfg.head_dim}, "
                        f"FFN {cfg.ffn}, vocab {cfg.vocab}, random-init {cfg.wtype} weights",
            "batch": cfg.batch,
            "kv_prefill": cfg.prefill,
            "positions": f"{cfg.prefill}..{cfg.prefill + steps - 1}",
            "path": "megakernel (1 persistent launch per step)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (None if traffic_bytes is None
                        else round(traffic_bytes / (avg_launch_ms * 1e-3) / 1e9, 1)),
        },
        "traffic_bytes_per_launch": None if traffic_bytes is None else int(traffic_bytes),
        "kernel": kname,
        "algorithmic_bytes_per_step": int(avg_bytes),
        "launches_per_step": info.launches_per_step,
        "step_ms_p10_p50_p90": [round(sorted(per)[int(q * (steps - 1))], 4) for q in (0.1, 0.5, 0.9)],
    }
    if not args.no_multistep:
        ms_m, ids_m = time_multistep(cfg, weights, kv_host, steps, warmup)
        out["multistep_one_launch"] = {
            "steps_per_launch": steps,
            "ms_per_step": round(ms_m, 4),
            "tokens_per_s": round(cfg.batch / (ms_m * 1e-3), 2),
            "hbm_gbs": round(avg_bytes / (ms_m * 1e-3) / 1e9, 1),
            "same_final_ids": ids_m == ids,
        }
        log(f"[bench] multistep: {ms_m:.4f} ms/step in one launch of {steps}")
    if not args.no_scenario and cfg.batch == 1:
        out["scenario_in64_out12"] = time_prompt_scenario(cfg, weights)
        log(f"[bench] in64/out12: {out['scenario_in64_out12']}")
    if not args.no_ablation:
        for key, graph in (("ablation_unfused", False), ("ablation_unfused_hipgraph", True)):
            ms_u, per_u, info_u, ids_u = time_path(cfg, weights, kv_host, "unfused", steps, warmup,
                                                   graph=graph)
            out[key] = {
                "ms_per_step": round(ms_u, 4),
                "tokens_per_s": round(cfg.batch / (ms_u * 1e-3), 2),
                "launches_per_step": info_u.launches_per_step,
                "hbm_gbs": round(avg_bytes / (ms_u * 1e-3) / 1e9, 1),
                "same_final_ids": ids_u == ids,
                "megakernel_speedup": round(ms_u / ms, 3),
            }
    if not args.no_cpu_baseline:
        t = time.time()
        out["cpu_baseline"] = cpu_baseline(cfg, weights, kv_host, args.cpu_sample_steps)
        log(f"[bench] cpu baseline took {time.time() - t:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
