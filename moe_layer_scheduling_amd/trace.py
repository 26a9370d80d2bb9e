"""Decode and summarise the per-task trace of etc_moe_layer (ETC_FLAG_TRACE).

Each record: task word (kind, layer, fields a-d), start of the claim on the 100 MHz
device clock, workgroup, ticks spent claiming / waiting on counters, ticks running.
"""

import json

import numpy as np

KINDS = {1: "R", 2: "S", 3: "GU", 4: "D", 5: "F", 6: "P"}
TICK_US = 0.01  # 100 MHz


def decode(records):
    r = np.asarray(records, dtype=np.uint64).reshape(-1, 4)
    task = r[:, 0]
    out = {
        "kind": (task & 15).astype(np.int32),
        "layer": ((task >> 4) & 15).astype(np.int32),
        "a": ((task >> 8) & 0x3FFF).astype(np.int32),
        "b": ((task >> 22) & 0x3FFF).astype(np.int32),
        "c": ((task >> 36) & 0x3FFF).astype(np.int32),
        "d": ((task >> 50) & 0x3FFF).astype(np.int32),
        "start": r[:, 1].astype(np.int64),
        "wg": (r[:, 2] & 0xFFFFFFFF).astype(np.int32),
        "wait": (r[:, 2] >> 32).astype(np.int64),
        "run": (r[:, 3] & 0xFFFFFFFF).astype(np.int64),
    }
    t0 = out["start"].min() if len(out["start"]) else 0
    out["start"] = out["start"] - t0
    return out


def summarize(records):
    """Per task kind: count, mean / total run and wait in microseconds, and the span."""
    d = decode(records)
    res = {}
    for k, name in KINDS.items():
        m = d["kind"] == k
        if not m.any():
            continue
        run, wait = d["run"][m] * TICK_US, d["wait"][m] * TICK_US
        res[name] = {"count": int(m.sum()), "run_mean_us": float(run.mean()),
                     "run_total_us": float(run.sum()), "wait_mean_us": float(wait.mean()),
                     "wait_total_us": float(wait.sum()),
                     "first_start_us": float(d["start"][m].min() * TICK_US),
                     "last_end_us": float(((d["start"] + d["wait"] + d["run"])[m]).max() * TICK_US)}
    end = (d["start"] + d["wait"] + d["run"]).max() * TICK_US if len(d["start"]) else 0.0
    res["span_us"] = float(end)
    res["workgroups"] = int(len(np.unique(d["wg"])))
    busy = float((d["run"].sum()) * TICK_US)
    res["busy_fraction"] = busy / (res["workgroups"] * end) if end else 0.0
    return res


def chrome_trace(records, path):
    """Write a Chrome trace (chrome://tracing, Perfetto): one row per workgroup."""
    d = decode(records)
    ev = []
    for i in range(len(d["kind"])):
        name = KINDS.get(int(d["kind"][i]), "?")
        args = {"layer": int(d["layer"][i]), "a": int(d["a"][i]), "b": int(d["b"][i]),
                "c": int(d["c"][i]), "d": int(d["d"][i])}
        if d["wait"][i] > 0:
            ev.append({"name": "wait", "ph": "X", "pid": 0, "tid": int(d["wg"][i]),
                       "ts": d["start"][i] * TICK_US, "dur": d["wait"][i] * TICK_US})
        ev.append({"name": name, "ph": "X", "pid": 0, "tid": int(d["wg"][i]),
                   "ts": (d["start"][i] + d["wait"][i]) * TICK_US, "dur": d["run"][i] * TICK_US,
                   "args": args})
    with open(path, "w") as f:
        json.dump({"traceEvents": ev}, f)
