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


def time_path(cfg, weights, kv_host, path, steps, warmup, graph=False, cold_mib=0):
    """Returns (ms per step from events around the whole timed region, per-launch durations ms,
    model info, final token ids). graph=True: each timed step is one hipGraph replay of the step's
    launches (captured beforehand, one graph per position, since the position is a launch argument).
    cold_mib > 0: before every step a kernel writes a scratch buffer of that size, evicting the
    model from the GPU's caches; each step is then timed by its own pair of events and the
    returned ms per step is their mean (the writes are not counted)."""
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
    flush = torch.empty((cold_mib << 20) // 4, dtype=torch.float32, device="cuda") if cold_mib else None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev_begin = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if cold_mib else None
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i))
            ev_begin[i].record(stream)
        if graph:
            graphs[i].replay()
        else:
            model.step(kv, tok, cfg.prefill + i, next_out=tok)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    model.sync()
    if flush is not None:
        per = [ev_begin[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        total = sum(per)
        del flush
    else:
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
    each (best of `reps`) and how far the two runs' tokens agree."""
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
    outs, lgs = {}, {}
    for _ in range(reps):
        for mode in ("hybrid", "decode_only"):
            kv = model.kv(1, max_seq)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            lg = torch.empty((n_out, 1, cfg.vocab), dtype=torch.float32, device="cuda")
            ev[0].record(stream)
            if mode == "hybrid":
                nxt = model.prefill(kv, prompt, 0)
            else:
                nxt = torch.empty(1, dtype=torch.int32, device="cuda")
                for i in range(n_in):
                    model.step(kv, prompt[i:i + 1], i, next_out=nxt)
            out = model.steps(kv, nxt, n_in, n_out, logits=lg)
            ev[1].record(stream)
            torch.cuda.synchronize()
            model.sync()
            best[mode] = min(best[mode], ev[0].elapsed_time(ev[1]))
            outs[mode] = out.cpu().numpy().ravel().tolist()
            lgs[mode] = lg.cpu().numpy()[:, 0].astype(np.float64)
            kv.close()
    model.close()
    torch.cuda.empty_cache()
    # The two runs agree on their tokens until the first step whose top-2 logit margin is within
    # their rounding difference (the prompt's KV rows are computed by different kernels); the
    # oracle parity of both paths at this width is a GPU test. Reported: where they part, and
    # how close the two runs' logits are at the first output step, which both reach from the
    # same prompt.
    a, b = outs["hybrid"], outs["decode_only"]
    first = next((i for i in range(n_out) if a[i] != b[i]), None)
    res = {"input_tokens": n_in, "output_tokens": n_out,
           "hybrid_ms": round(best["hybrid"], 3), "decode_only_ms": round(best["decode_only"], 3),
           "hybrid_speedup": round(best["decode_only"] / best["hybrid"], 3),
           "output_tokens_equal_until": n_out if first is None else first,
           "step0_max_abs_logit_diff": round(float(np.max(np.abs(lgs["hybrid"][0] - lgs["decode_only"][0]))), 6)}
    if first is not None:
        top2 = np.sort(lgs["hybrid"][first])[-2:]
        res["hybrid_top2_margin_at_first_difference"] = round(float(top2[1] - top2[0]), 6)
    return res


def profiled_traffic(key, kernel_name):
    """Per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from the committed
    rocprofv3 summary of this workload (profiles/megakernel_<key>.json, key = name_b<batch>), or
    None when the kernel sources changed since."""
    from persistent_decode_megakernel_amd import profile_summary
    path = os.path.join(ROOT, "profiles", f"megakernel_{key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel_name or rec.get("source_hash") != profile_summary.source_hash():
        return None
    return float(rec["traffic_bytes_per_launch"])


def cpu_baseline(cfg, weights, kv_host, sample_steps, threads=16):
    """The oracle as it stands, in its float32 mode (weights converted to float32 once, before
    the timed region), on a bounded sample of the same workload: the first `sample_steps` greedy
    decode steps of the full model from the same prefilled cache and first token, with the BLAS
    thread pool limited to `threads` (the host cores a GPU's share of the box provides)."""
    import numpy as np
    import oracle
    from persistent_decode_megakernel_amd import synth

    params, wn = synth.oracle_inputs(weights)
    pos = cfg.prefill
    kv = synth.bf16_to_numpy_bits(kv_host[..., :pos + sample_steps + 1, :]).copy()
    tok = synth.make_tokens(cfg, 0)[:, 0].numpy()
    dec = oracle.Decoder(params, wn, dtype=np.float32, cache_bytes=64 << 30)
    host_cores = len(os.sched_getaffinity(0))
    used = min(threads, host_cores)
    limiter = None
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=used, user_api="blas")
    except Exception:  # threadpoolctl absent: BLAS keeps its own thread count
        used = int(os.environ.get("OMP_NUM_THREADS", host_cores))
    t = time.perf_counter()
    dec.step(kv.copy(), tok, pos)  # converts every weight matrix once (not timed)
    t_conv = time.perf_counter() - t
    t = time.perf_counter()
    for i in range(sample_steps):
        logits = dec.step(kv, tok, pos + i)
        tok = oracle.argmax_lowest(logits)
    t_step = (time.perf_counter() - t) / sample_steps
    if limiter is not None:
        limiter.restore_original_limits()
    return {
        "value": round(cfg.batch / t_step, 4),
        "unit": "tokens/s",
        "cores": used,
        "kind": "oracle",
        "sample": (f"{sample_steps} greedy decode steps of the full {cfg.name} model at positions "
                   f"{pos}..{pos + sample_steps - 1}, {t_step:.2f} s per step: the oracle's "
                   f"float32 numpy matrix-vector products on {used} BLAS threads (host has "
                   f"{host_cores} cores), weights converted to float32 once beforehand "
                   f"({t_conv:.1f} s, not timed)"),
    }


def kernel_name(cfg, info):
    """the megakernel instance the model runs (query heads per attention pass from the library)"""
    wt = {"bf16": 0, "int8": 1, "int4": 2}[cfg.wtype]
    return (f"amk_megakernel_w{wt}_h{cfg.head_dim}_q{info.heads_per_pass}"
            + ("_b" if cfg.batch > 1 else ""))


def measure(cfg, weights, kv_host, steps, warmup, ablation=True, graph_ablation=False,
            cold_mib=0, profile_key=None):
    """Megakernel steps of one workload with its roofline: algorithmic bytes per launch (weights,
    norm gains, scales, embedding rows and the KV rows each step reads) over the mean launch time
    from events on the launch stream; and, optionally, the unfused ablation on the same inputs."""
    ms, per, info, ids = time_path(cfg, weights, kv_host, "megakernel", steps, warmup,
                                   cold_mib=cold_mib)
    kname = kernel_name(cfg, info)
    traffic_bytes = profiled_traffic(profile_key or f"{cfg.name}_b{cfg.batch}", kname)
    weight_bytes = info.weight_bytes + 2 * cfg.hidden * cfg.batch  # + embedding rows
    ctxs = [cfg.prefill + i + 1 for i in range(steps)]
    avg_bytes = sum(weight_bytes + kv_bytes_step(cfg, c) for c in ctxs) / steps
    avg_launch_ms = sum(per) / steps  # one launch per step
    achieved = avg_bytes / (avg_launch_ms * 1e-3) / 1e9
    res = {
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(cfg.batch / (ms * 1e-3), 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (None if traffic_bytes is None
                        else round(traffic_bytes / (avg_launch_ms * 1e-3) / 1e9, 1)),
        },
        "kernel": kname,
        "algorithmic_bytes_per_step": int(avg_bytes),
        "traffic_bytes_per_launch": None if traffic_bytes is None else int(traffic_bytes),
        "launches_per_step": info.launches_per_step,
        "step_ms_p10_p50_p90": [round(sorted(per)[int(q * (steps - 1))], 4) for q in (0.1, 0.5, 0.9)],
        "positions": f"{cfg.prefill}..{cfg.prefill + steps - 1}",
        "batch": cfg.batch,
        "_ids": ids,
    }
    if ablation:
        variants = (("ablation_unfused", False),) + ((("ablation_unfused_hipgraph", True),)
                                                     if graph_ablation else ())
        for key, graph in variants:
            ms_u, per_u, info_u, ids_u = time_path(cfg, weights, kv_host, "unfused", steps, warmup,
                                                   graph=graph, cold_mib=cold_mib)
            res[key] = {
                "ms_per_step": round(ms_u, 4),
                "tokens_per_s": round(cfg.batch / (ms_u * 1e-3), 2),
                "launches_per_step": info_u.launches_per_step,
                "hbm_gbs": round(avg_bytes / (ms_u * 1e-3) / 1e9, 1),
                "same_final_ids": ids_u == ids,
                "megakernel_speedup": round(ms_u / ms, 3),
            }
    return res


# the other workloads measured in the same run (BASELINE configs and the batch-8 matrix-core step)
EXTRA = [("smollm2_135m", {}), ("smollm2_135m_cold", {"cold_mib": 1024}), ("tinyllama_1b", {}),
         ("llama2_7b_w8a16", {}), ("llama2_7b_b8", {})]


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
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --workload, not the other configurations")
    ap.add_argument("--batch", type=int, default=0,
                    help="override the workload's batch (sequences per step, 1..16)")
    ap.add_argument("--cpu-sample-steps", type=int, default=8)
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

    head = measure(cfg, weights, kv_host, steps, warmup, ablation=not args.no_ablation,
                   graph_ablation=True)
    ids = head.pop("_ids")
    out = {
        "metric": "decode tokens/s at batch 1 + achieved HBM GB/s as % of 8 TB/s peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
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
            "positions": head["positions"],
            "path": "megakernel (1 persistent launch per step)",
        },
        "roofline": head["roofline"],
    }
    for k in ("traffic_bytes_per_launch", "kernel", "algorithmic_bytes_per_step",
              "launches_per_step", "step_ms_p10_p50_p90", "ablation_unfused",
              "ablation_unfused_hipgraph"):
        if k in head:
            out[k] = head[k]
    if not args.no_multistep:
        ms_m, ids_m = time_multistep(cfg, weights, kv_host, steps, warmup)
        out["multistep_one_launch"] = {
            "steps_per_launch": steps,
            "ms_per_step": round(ms_m, 4),
            "tokens_per_s": round(cfg.batch / (ms_m * 1e-3), 2),
            "hbm_gbs": round(head["algorithmic_bytes_per_step"] / (ms_m * 1e-3) / 1e9, 1),
            "same_final_ids": ids_m == ids,
        }
        log(f"[bench] multistep: {ms_m:.4f} ms/step in one launch of {steps}")
    if not args.no_scenario and cfg.batch == 1:
        out["scenario_in64_out12"] = time_prompt_scenario(cfg, weights)
        log(f"[bench] in64/out12: {out['scenario_in64_out12']}")
    if not args.no_cpu_baseline:
        t = time.time()
        out["cpu_baseline"] = cpu_baseline(cfg, weights, kv_host, args.cpu_sample_steps)
        log(f"[bench] cpu baseline took {time.time() - t:.1f}s")
    if not args.no_extra and not args.batch and args.workload == "llama2_7b":
        out["workloads"] = {}
        cache = {}
        for key, opt in EXTRA:
            name = key.replace("_cold", "")
            wcfg = synth.get_config(name)
            t = time.time()
            w_key = (wcfg.cfg_id, wcfg.wtype)
            if w_key == (cfg.cfg_id, cfg.wtype):
                wts = weights  # the batch-8 workload shares the headline model's weights
            else:
                if w_key not in cache:
                    cache.clear()
                    cache[w_key] = synth.make_weights(wcfg, 0, threads=16)
                wts = cache[w_key]
            kvh = synth.make_kv(wcfg, wcfg.prefill + max(steps, warmup) + 1, 0, threads=16)
            # counters are taken on warm runs: the cold variant reports none of its own
            pkey = f"{wcfg.name}_b{wcfg.batch}" + ("_cold" if opt.get("cold_mib") else "")
            res = measure(wcfg, wts, kvh, steps, warmup, profile_key=pkey, **opt)
            res.pop("_ids")
            res["workload"] = (f"{wcfg.name}: {wcfg.n_layers} layers, hidden {wcfg.hidden}, "
                               f"{wcfg.n_heads}/{wcfg.n_kv_heads} heads, head_dim {wcfg.head_dim}, "
                               f"FFN {wcfg.ffn}, vocab {wcfg.vocab}{', tied' if wcfg.tied else ''}, "
                               f"{wcfg.wtype}, KV prefill {wcfg.prefill}"
                               + (f", {opt['cold_mib']} MiB written between steps" if opt.get("cold_mib") else ""))
            out["workloads"][key] = res
            del kvh
            log(f"[bench] {key}: {res['ms_per_step']} ms/step, frac {res['roofline']['frac']} "
                f"({time.time() - t:.1f}s)")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
