"""Summaries of the megakernel's task trace (see amk_trace_enable) and export to the Chrome /
Perfetto JSON trace format.

Each task carries four 100 MHz wall-clock stamps: start of its dependency wait, wait done,
input staged (GEMV tasks), end. Phases are (layer, task kind)."""
from __future__ import annotations

import json
from collections import defaultdict
from typing import Dict

import numpy as np

from .blob import M_D, M_GU, M_LM, M_O, M_QKV, T_ARGMAX, T_ATTN, T_GEMV, Blob

KIND = {(T_GEMV, M_QKV): "qkv", (T_GEMV, M_O): "o", (T_GEMV, M_GU): "gateup",
        (T_GEMV, M_D): "down", (T_GEMV, M_LM): "lm_head"}
TICK_US = 0.01  # 100 MHz


def task_table(blob: Blob):
    rows = []
    for cu, v in enumerate(blob.per_cu):
        for t in v:
            kind = KIND.get((int(t["type"]), int(t["mat"])),
                            "attn" if t["type"] == T_ATTN else "argmax")
            rows.append((int(t["id"]), cu, int(t["layer"]), kind))
    rows.sort()
    return rows


def summarize(blob: Blob, trace: np.ndarray) -> Dict:
    n = blob.hdr.n_tasks
    ts = trace[: 4 * n].reshape(n, 4).astype(np.int64)
    xcc = trace[4 * n: 4 * n + blob.hdr.n_cu]
    t0 = ts[:, 0].min()
    rows = task_table(blob)
    phases = defaultdict(list)
    for tid, cu, layer, kind in rows:
        phases[(layer if kind not in ("lm_head", "argmax") else 10 ** 6, kind)].append(tid)
    out = {"step_us": float((ts[:, 3].max() - t0) * TICK_US), "phases": {}}
    kinds = defaultdict(lambda: np.zeros(4))
    for key, ids in sorted(phases.items()):
        a = ts[ids]
        wait = (a[:, 1] - a[:, 0]) * TICK_US
        stage = np.where(a[:, 2] > 0, a[:, 2] - a[:, 1], 0) * TICK_US
        body = (a[:, 3] - np.where(a[:, 2] > 0, a[:, 2], a[:, 1])) * TICK_US
        span = (a[:, 3].max() - a[:, 0].min()) * TICK_US
        out["phases"][f"{key[0]}:{key[1]}"] = {
            "tasks": len(ids), "span_us": float(span), "wait_mean_us": float(wait.mean()),
            "stage_mean_us": float(stage.mean()), "body_mean_us": float(body.mean()),
            "body_max_us": float(body.max()),
            "first_start_us": float((a[:, 0].min() - t0) * TICK_US),
            "last_end_us": float((a[:, 3].max() - t0) * TICK_US)}
        k = kinds[key[1]]
        k += np.array([wait.sum(), stage.sum(), body.sum(), len(ids)])
    out["by_kind_mean_us"] = {k: {"wait": v[0] / v[3], "stage": v[1] / v[3], "body": v[2] / v[3]}
                              for k, v in kinds.items()}
    out["xcc_of_workgroup"] = [int(x) for x in xcc[:32]]
    return out


def to_chrome_json(blob: Blob, trace: np.ndarray, path: str) -> None:
    n = blob.hdr.n_tasks
    ts = trace[: 4 * n].reshape(n, 4).astype(np.int64)
    t0 = ts[:, 0].min()
    ev = []
    for tid, cu, layer, kind in task_table(blob):
        a = ts[tid]
        ev.append({"name": f"wait {kind}", "ph": "X", "pid": 0, "tid": cu,
                   "ts": (a[0] - t0) * TICK_US, "dur": (a[1] - a[0]) * TICK_US})
        ev.append({"name": f"{kind} L{layer}", "ph": "X", "pid": 0, "tid": cu,
                   "ts": (a[1] - t0) * TICK_US, "dur": (a[3] - a[1]) * TICK_US})
    with open(path, "w") as f:
        json.dump({"traceEvents": ev}, f)
