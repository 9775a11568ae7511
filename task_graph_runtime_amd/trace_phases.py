"""Per-phase summary of a traced decode step (``TGraph.set_trace`` /
``read_trace``).  For each layer asked for, the tasks of one type form a
phase (the q/k/v tiles, the attention splits, the O tiles, ...), listed in
the order they start, with

* gap  -- from the previous phase's last task end to this phase's first start;
* span -- from the phase's first start to its last end;
* task -- the mean task duration, start to stores complete, over all of the
  phase's tasks and over those that set their marks (an attention slot with no
  split to run sets none);
* pro / body / epi -- a task's two marks cut it into prologue (start to its
  input staged), body (the weight or key/value stream) and epilogue (the
  reduction and stores); a task that sets only the second mark (the
  matrix-core tiles) has its body counted from its start.

Run as a module on a GPU, it builds the decoder of a named shape on seeded
synthetic inputs, runs a few steps, traces one and prints the tables:

    python -m task_graph_runtime_amd.trace_phases --config qwen3_8b --layers 5 20
"""
from __future__ import annotations

import numpy as np

from . import _binding as _b

TYPE_NAMES = {getattr(_b, n): n[5:].lower() for n in dir(_b) if n.startswith("TASK_")}


def phase_table(records: np.ndarray, ticks_per_us: float, graph: dict, layer: int) -> list:
    """Rows (dicts) of one layer's phases; times in microseconds from the
    layer's first task start.  `records`, `ticks_per_us`: ``read_trace()``;
    `graph`: ``export()``."""
    tt, tl = graph["task_type"], graph["task_layer"]
    sel = records[tl[records["task"]] == layer]
    sel = sel[tt[sel["task"]] != _b.TASK_EMPTY]
    if len(sel) == 0:
        return []
    t0 = float(sel["t_start"].min())

    def us(x):
        return (np.asarray(x, np.float64) - t0) / ticks_per_us

    kinds = sorted({int(tt[t]) for t in sel["task"]}, key=lambda k: us(sel[tt[sel["task"]] == k]["t_start"]).min())
    rows, prev_end = [], None
    for k in kinds:
        r = sel[tt[sel["task"]] == k]
        st, en = us(r["t_start"]), us(r["t_end"])
        m0, m1 = r["t_mark"][:, 0], r["t_mark"][:, 1]
        h0, h1 = m0 > 0, m1 > 0
        row = {"phase": TYPE_NAMES.get(k, str(k)), "n": len(r), "n_marked": int(h1.sum()),
               "gap": None if prev_end is None else float(st.min() - prev_end),
               "start": float(st.min()), "end": float(en.max()), "span": float(en.max() - st.min()),
               "task": float((en - st).mean())}
        if h1.any():
            row["task_marked"] = float((en[h1] - st[h1]).mean())
            both = h0 & h1
            if both.any():
                row["pro"] = float((us(m0[both]) - st[both]).mean())
                row["body"] = float((us(m1[both]) - us(m0[both])).mean())
            else:
                row["body"] = float((us(m1[h1]) - st[h1]).mean())
            row["epi"] = float((en[h1] - us(m1[h1])).mean())
        rows.append(row)
        prev_end = float(en.max())
    return rows


def markdown(rows: list) -> str:
    """The rows as a markdown table (µs)."""
    f = lambda v: "" if v is None else f"{v:.1f}"
    out = ["| phase | tasks (marked) | gap | span | task (marked) | pro | body | epi |", "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        task = f(r["task"]) + (f" ({f(r['task_marked'])})" if "task_marked" in r and r["n_marked"] != r["n"] else "")
        out.append(f"| {r['phase']} | {r['n']} ({r['n_marked']}) | {f(r['gap'])} | {f(r['span'])} | {task} | "
                   f"{f(r.get('pro'))} | {f(r.get('body'))} | {f(r.get('epi'))} |")
    return "\n".join(out)


def layer_starts(records: np.ndarray, ticks_per_us: float, graph: dict) -> dict:
    """First task start of every layer, in µs from the step's first start."""
    tl = graph["task_layer"]
    t0 = float(records["t_start"].min())
    out = {}
    for r in records:
        layer = int(tl[r["task"]])
        t = (float(r["t_start"]) - t0) / ticks_per_us
        if layer not in out or t < out[layer]:
            out[layer] = t
    return out


def main(argv=None) -> int:
    import argparse
    import json
    import torch
    import synth
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", default="qwen3_8b")
    ap.add_argument("--layers", type=int, nargs="+", default=[5, 20], help="layers to show (-1: the LM head)")
    ap.add_argument("--params", default="{}", help="build parameters (JSON), as in bench.py")
    ap.add_argument("--prepared", action="store_true", help="batch > 1: weights prepared by mpk_prepare_weights")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args(argv)
    s = synth.SHAPES[args.config]
    inp = synth.make_inputs(s, seed=args.seed, device="cuda")
    kv = inp["kv"]
    g = _b.TGraph(s.cfg(), s.batch, s.page_size, json.loads(args.params))
    w = _b.Weights(inp["weights"])
    if args.prepared:
        w = _b.PreparedWeights(g, w)
    kvs = _b.KV(kv["k_pool"], kv["v_pool"], kv["page_table"].cuda())
    ids, lens = inp["token_ids"].cuda(), inp["seq_lens"].cuda()
    logits = torch.empty((s.batch, s.vocab), device="cuda")
    nxt = torch.empty((s.batch,), device="cuda", dtype=torch.int32)
    for _ in range(3):
        g.decode_step(w, ids, kvs, lens, logits, nxt)
    g.set_trace(True)
    g.decode_step(w, ids, kvs, lens, logits, nxt)
    torch.cuda.synchronize()
    rec, tpu = g.read_trace()
    ex = g.export()
    starts = layer_starts(rec, tpu, ex)
    step = (float(rec["t_done"].max()) - float(rec["t_start"].min())) / tpu
    print(f"{args.config}: traced step {step:.1f} us (first start to last trigger), {len(rec)} task records")
    for layer in args.layers:
        nxt_start = starts.get(layer + 1) if layer >= 0 else None
        period = "" if nxt_start is None else f", layer period {nxt_start - starts[layer]:.1f} us"
        print(f"\nlayer {layer}{period}\n")
        print(markdown(phase_table(rec, tpu, ex, layer)))
    g.close()
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
