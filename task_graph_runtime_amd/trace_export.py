"""Export of the in-kernel trace (``TGraph.read_trace``) in the Chrome
trace-event JSON format, which the Perfetto UI (ui.perfetto.dev) and
chrome://tracing open.

One track per worker (the compute unit's workgroup).  Per task record:

* ``wait`` -- from the moment the worker started polling for the task to the
  moment it saw the task's event fire (or its JIT ring slot);
* the task itself, named by its type, layer and coordinates, from its start
  to the moment its stores completed; with the task's two marks inside it
  (set by the projection tiles and the attention splits) it is cut into
  ``prologue`` / ``body`` / ``epilogue`` child slices;
* ``trigger`` -- the arrival at its triggering event, including the empty
  tasks and JIT hand-overs the arrival resolves.

Optionally (``flows=True``) an arrow from the producer whose trigger finished
last to each consumer of an event: the arrival that released the consumer.
Times are microseconds from the earliest start in the step.
"""
from __future__ import annotations

import json

import numpy as np

from . import _binding as _b

TYPE_NAMES = {getattr(_b, n): n[5:].lower() for n in dir(_b) if n.startswith("TASK_")}


def _name(graph: dict, t: int) -> str:
    ty = int(graph["task_type"][t])
    layer = int(graph["task_layer"][t])
    c = graph["task_coords"][t]
    nm = TYPE_NAMES.get(ty, f"type{ty}")
    where = f"L{layer}" if layer >= 0 else "head"
    return f"{nm} {where} ({int(c[0])},{int(c[1])},{int(c[2])})"


def chrome_trace(records: np.ndarray, ticks_per_us: float, graph: dict, flows: bool = False) -> dict:
    """The trace-event document (a dict) of one traced step.  `records`,
    `ticks_per_us`: ``TGraph.read_trace()``; `graph`: ``TGraph.export()``."""
    if len(records) == 0:
        return {"traceEvents": [], "displayTimeUnit": "ns"}
    t0 = int(min(int(r) for r in records["t_start"]))

    def us(x) -> float:
        return (int(x) - t0) / ticks_per_us

    ev = []
    workers = sorted(set(int(w) for w in records["worker"]))
    ev.append({"ph": "M", "pid": 0, "name": "process_name", "args": {"name": "mpk_megakernel (one step)"}})
    for w in workers:
        ev.append({"ph": "M", "pid": 0, "tid": w, "name": "thread_name", "args": {"name": f"worker {w:3d}"}})
        ev.append({"ph": "M", "pid": 0, "tid": w, "name": "thread_sort_index", "args": {"sort_index": w}})
    done_at = {}
    for r in records:
        t = int(r["task"])
        w = int(r["worker"])
        ts, te, td, tw = us(r["t_start"]), us(r["t_end"]), us(r["t_done"]), us(r["t_wait"])
        args = {"task": t, "dep_event": int(graph["task_dep"][t]), "trig_event": int(graph["task_trig"][t]),
                "mode": ("AOT", "JIT", "EMPTY")[int(graph["task_mode"][t])]}
        if ts > tw:
            ev.append({"ph": "X", "pid": 0, "tid": w, "name": "wait", "cat": "wait", "ts": tw, "dur": ts - tw,
                       "args": {"for": t}})
        ev.append({"ph": "X", "pid": 0, "tid": w, "name": _name(graph, t), "cat": TYPE_NAMES.get(int(graph["task_type"][t]), "task"),
                   "ts": ts, "dur": max(0.0, te - ts), "args": args})
        m0, m1 = int(r["t_mark"][0]), int(r["t_mark"][1])
        if m0 and m1 and int(r["t_start"]) <= m0 <= m1 <= int(r["t_end"]):
            a, b = us(m0), us(m1)
            for nm, s0, s1 in (("prologue", ts, a), ("body", a, b), ("epilogue", b, te)):
                ev.append({"ph": "X", "pid": 0, "tid": w, "name": nm, "cat": "phase", "ts": s0, "dur": max(0.0, s1 - s0)})
        if td > te:
            ev.append({"ph": "X", "pid": 0, "tid": w, "name": "trigger", "cat": "trigger", "ts": te, "dur": td - te,
                       "args": {"event": int(graph["task_trig"][t])}})
        done_at[t] = (td, w)
    if flows:
        # the producer of each event whose trigger finished last released its consumers
        last_prod = {}
        for t, (td, w) in done_at.items():
            e = int(graph["task_trig"][t])
            if e not in last_prod or td > last_prod[e][0]:
                last_prod[e] = (td, w, t)
        fid = 0
        for r in records:
            t = int(r["task"])
            e = int(graph["task_dep"][t])
            if e in last_prod:
                td, w, p = last_prod[e]
                fid += 1
                ev.append({"ph": "s", "pid": 0, "tid": w, "name": "release", "cat": "event", "id": fid, "ts": td})
                ev.append({"ph": "f", "pid": 0, "tid": int(r["worker"]), "name": "release", "cat": "event", "id": fid,
                           "ts": us(r["t_start"]), "bp": "e"})
    return {"traceEvents": ev, "displayTimeUnit": "ns"}


def write_chrome_trace(path: str, records: np.ndarray, ticks_per_us: float, graph: dict, flows: bool = False) -> int:
    """Write the trace-event JSON of one traced step to `path`; returns the
    number of trace events written."""
    doc = chrome_trace(records, ticks_per_us, graph, flows)
    with open(path, "w") as f:
        json.dump(doc, f)
    return len(doc["traceEvents"])
