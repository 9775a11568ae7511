"""The in-kernel runtime protocol, simulated on the CPU (protocol_sim) over
graphs the library builds: every scheduling policy, fusion on and off, k-splits,
the operator-level graph and a mixture-of-experts decoder, several steps on
never-reset counters under random timings -- and graphs broken on purpose,
which the simulator must reject."""
import numpy as np
import pytest

import synth
import task_graph_runtime_amd as mpk
from oracle import tgraph as tg
from task_graph_runtime_amd.protocol_sim import ProtocolError, simulate, TICKS_PER_UNIT
from task_graph_runtime_amd import trace_export


def export(shape, B, params):
    g = mpk.TGraph(shape.cfg(), B, shape.page_size, params, host_only=True)
    ex = g.export()
    ex["params"] = g.header()["params"]
    g.close()
    return ex


def region_order(shape, B, g):
    """The relation the regions define, independent of the library's events:
    for every task (linear index), the tasks whose output region overlaps one
    of its input regions (the oracle's brute-force overlap on the oracle's own
    decomposition with the same build parameters), mapped to linear indices."""
    p = g["params"]
    prm = tg.Params(W=p["n_workers"], S_sched=p["n_sched_waves"], q=p["quantum"], T_qkv=p["t_qkv"], T_o=p["t_o"],
                    T_gu=p["t_gu"], T_down=p["t_down"], T_lm=p["t_lm"], S_attn=p["s_attn"],
                    jit_attn=p["attn_jit"] == 1, jit_all=p["attn_jit"] == 3, K_qkv=p["k_qkv"], K_o=p["k_o"],
                    K_down=p["k_down"], coarse=p["coarse_events"] == 1, fusion=p["fusion_order"],
                    T_router=p["t_router"] or 1, T_egu=p["t_egu"] or 1, T_edown=p["t_edown"] or 1)
    _, tasks = tg.build(shape.cfg(), B, shape.page_size, prm)
    P = tg.producer_sets(tasks)
    lin = {int(o): i for i, o in enumerate(g["task_orig"]) if o >= 0}
    out = [set() for _ in range(len(g["task_orig"]))]
    for c, ps in enumerate(P):
        out[lin[c]] = {lin[q] for q in ps}
    return out


TINY = synth.SHAPES["tiny"]

CASES = [
    ("tiny b1 AOT", TINY, 1, dict(n_workers=8, s_attn=4)),
    ("tiny b1 hybrid", TINY, 1, dict(n_workers=8, n_sched_waves=2, s_attn=4, attn_jit=1)),
    ("tiny b1 pure JIT", TINY, 1, dict(n_workers=9, n_sched_waves=3, s_attn=4, attn_jit=3)),
    ("tiny b3 AOT k-split", TINY, 3, dict(n_workers=12, s_attn=6, k_qkv=2, k_o=2, k_down=3, t_qkv=8, t_o=6, t_down=6)),
    ("tiny b3 hybrid", TINY, 3, dict(n_workers=12, n_sched_waves=4, s_attn=6, attn_jit=1)),
    ("tiny b3 pure JIT", TINY, 3, dict(n_workers=10, n_sched_waves=5, s_attn=6, attn_jit=3)),
    ("tiny b1 no fusion", TINY, 1, dict(n_workers=8, s_attn=4, fusion_order=1)),
    ("tiny b3 no fusion hybrid", TINY, 3, dict(n_workers=8, n_sched_waves=2, s_attn=4, fusion_order=1, attn_jit=1)),
    ("tiny b3 no fusion pure JIT", TINY, 3, dict(n_workers=8, n_sched_waves=4, s_attn=4, fusion_order=1, attn_jit=3)),
    ("tiny b1 operator-level", TINY, 1, dict(n_workers=8, s_attn=4, coarse_events=1)),
    ("tiny b3 operator-level hybrid", TINY, 3, dict(n_workers=8, n_sched_waves=2, s_attn=4, coarse_events=1, attn_jit=1)),
    ("tiny moe b1", synth.SHAPES["tiny_moe"], 1, dict(n_workers=8, s_attn=4)),
    ("tiny moe b4 hybrid", synth.SHAPES["tiny_moe"], 4, dict(n_workers=8, n_sched_waves=2, s_attn=4, attn_jit=1)),
]


@pytest.mark.parametrize("name,shape,B,params", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_protocol_terminates_in_order(name, shape, B, params, seed):
    g = export(shape, B, params)
    st = simulate(g, steps=3, seed=seed, must_follow=region_order(shape, B, g))
    assert st.steps == 3
    if g["params"]["attn_jit"] in (1, 3):
        assert st.jit_tasks == 3 * int(np.sum(g["task_mode"] == 1))


@pytest.mark.parametrize("seed", [0, 1])
def test_protocol_extreme_timings(seed):
    """Arrivals and polls far slower than tasks, and the reverse."""
    g = export(TINY, 3, dict(n_workers=8, n_sched_waves=2, s_attn=6, attn_jit=1))
    simulate(g, steps=2, seed=seed, task_time=(0.01, 0.02), op_time=(1.0, 50.0))
    simulate(g, steps=2, seed=seed, task_time=(1.0, 500.0), op_time=(0.001, 0.01))


def test_protocol_full_size_graph():
    """A full-size graph: the Qwen3-0.6B shape at batch 1 with the default
    build (256 workers, every task AOT, two-level events)."""
    g = export(synth.SHAPES["qwen3_0p6b"], 1, {})
    assert np.any(g["event_counts"] >= 64)
    st = simulate(g, steps=2, seed=0)
    assert st.steps == 2


def test_protocol_full_size_hybrid_batch16():
    g = export(synth.SHAPES["qwen3_0p6b"].with_(n_layers=4), 16, dict(attn_jit=1))
    assert g["params"]["n_sched_waves"] > 0
    st = simulate(g, steps=2, seed=1)
    assert st.jit_tasks > 0


# ---- graphs broken on purpose: the simulator must reject every one

def _base():
    return export(TINY, 3, dict(n_workers=8, n_sched_waves=2, s_attn=6, attn_jit=1))


def _real_consumer_event(g):
    """An event whose consumers are non-empty tasks and whose producers are
    several non-empty tasks (a projection's event)."""
    mode, trig = g["task_mode"], g["task_trig"]
    for e in range(len(g["event_counts"])):
        lo, hi = g["event_first"][e], g["event_last"][e]
        if hi < lo or not np.all(mode[lo:hi + 1] == 0):
            continue
        prod = np.nonzero(trig == e)[0]
        if len(prod) >= 3 and np.all(mode[prod] == 0):
            return e
    raise AssertionError("no such event")


def test_rejects_count_too_high():
    g = _base()
    e = _real_consumer_event(g)
    g["event_counts"] = g["event_counts"].copy()
    g["event_counts"][e] += 1          # one arrival more than there are producers: never fires
    with pytest.raises(ProtocolError, match="left waiting"):
        simulate(g, steps=1)


def test_rejects_count_too_low():
    g = _base()
    e = _real_consumer_event(g)
    g["event_counts"] = g["event_counts"].copy()
    g["event_counts"][e] -= 1          # fires one arrival early
    with pytest.raises(ProtocolError):
        for seed in range(20):
            simulate(g, steps=2, seed=seed)


def test_rejects_wrong_dependent_event():
    """A consumer pointed at an event that fires before its real producers
    finish: the regions' order catches it under some timing."""
    g = _base()
    ref = region_order(TINY, 3, g)
    e = _real_consumer_event(g)
    c = int(g["event_first"][e])
    earlier = int(g["task_dep"][np.nonzero(g["task_trig"] == e)[0][0]])   # a producer's own dependent event
    g["task_dep"] = g["task_dep"].copy()
    g["task_dep"][c] = earlier
    with pytest.raises(ProtocolError, match="before its producer"):
        for seed in range(20):
            simulate(g, steps=1, seed=seed, must_follow=ref)


def test_rejects_non_topological_aot_list():
    """Two AOT tasks of one worker in reverse dependency order: FIFO execution deadlocks."""
    g = export(TINY, 1, dict(n_workers=4, s_attn=4))
    aot, off = g["aot_tasks"].copy(), g["aot_offsets"]
    trig, dep = g["task_trig"], g["task_dep"]
    swapped = False
    for w in range(len(off) - 1):
        lst = aot[off[w]:off[w + 1]]
        for i in range(len(lst) - 1):
            a, b = lst[i], lst[i + 1]
            # b waits (directly) on the event a triggers
            if dep[b] == trig[a]:
                lst[i], lst[i + 1] = b, a
                swapped = True
                break
        if swapped:
            break
    assert swapped
    g["aot_tasks"] = aot
    with pytest.raises(ProtocolError, match="left waiting"):
        simulate(g, steps=1)


def test_rejects_duplicate_jit_hand_over():
    """A JIT event that claims one consumer more than its range: a task is
    dealt twice (or a non-JIT task is dealt)."""
    g = _base()
    jit_ev = [e for e in range(len(g["event_counts"])) if g["event_flags"][e] & 1]
    assert jit_ev
    e = jit_ev[0]
    g["event_last"] = g["event_last"].copy()
    g["event_last"][e] += 1
    with pytest.raises(ProtocolError):
        simulate(g, steps=1)


@pytest.mark.parametrize("name,B,params", [("qwen3_8b", 1, {}), ("qwen3_8b_b16", 16, dict(attn_jit=1)),
                                           ("qwen3_8b_b16", 16, dict(attn_jit=3))])
def test_protocol_bench_graphs(name, B, params):
    """The graphs of the benchmark shapes (8B, 36 layers, 46-49K tasks) at their
    default build and under the hybrid and pure-JIT policies."""
    g = export(synth.SHAPES[name], B, params)
    st = simulate(g, steps=2, seed=3)
    assert st.steps == 2


def test_perfetto_export_of_a_simulated_step(tmp_path):
    """The trace-event export on the schedule of a simulated step: one slice per
    non-empty task on its worker's track, no two overlapping on a track,
    waits and triggers around them, and every release arrow pointing forward."""
    g = export(TINY, 3, dict(n_workers=8, n_sched_waves=2, s_attn=6, attn_jit=1))
    st = simulate(g, steps=2, seed=5, trace=True)
    rec = st.trace
    real = np.nonzero(g["task_mode"] != 2)[0]
    assert sorted(rec["task"].tolist()) == real.tolist()
    path = tmp_path / "step.json"
    n = trace_export.write_chrome_trace(str(path), rec, TICKS_PER_UNIT, g, flows=True)
    import json
    doc = json.load(open(path))
    ev = doc["traceEvents"]
    assert len(ev) == n
    tasks = [e for e in ev if e["ph"] == "X" and e["cat"] not in ("wait", "trigger", "phase")]
    assert len(tasks) == len(real)
    assert all(e["args"]["task"] in set(real.tolist()) for e in tasks)
    by_w = {}
    for e in tasks:
        by_w.setdefault(e["tid"], []).append((e["ts"], e["ts"] + e["dur"]))
    for w, sl in by_w.items():
        sl.sort()
        assert all(a[1] <= b[0] + 1e-9 for a, b in zip(sl, sl[1:])), w
    s_ev = {e["id"]: e["ts"] for e in ev if e["ph"] == "s"}
    f_ev = {e["id"]: e["ts"] for e in ev if e["ph"] == "f"}
    assert s_ev and s_ev.keys() == f_ev.keys()
    assert all(s_ev[i] <= f_ev[i] + 1e-9 for i in s_ev)
    names = {e["name"].split()[0] for e in tasks}
    assert {"qkv", "attn", "oproj", "gateup", "down", "lmhead", "argmax"} <= names


def test_phase_table_of_a_simulated_step():
    """The per-phase summary (trace_phases) on the schedule of a simulated step:
    one row per task type of the layer, in start order, every non-empty task
    counted once, gaps measured from the previous phase's last end."""
    from task_graph_runtime_amd import trace_phases
    g = export(TINY, 3, dict(n_workers=8, n_sched_waves=2, s_attn=6, attn_jit=1))
    st = simulate(g, steps=1, seed=7, trace=True)
    rec = st.trace
    for layer in (0, 1, -1):
        rows = trace_phases.phase_table(rec, TICKS_PER_UNIT, g, layer)
        real = [t for t in np.nonzero(g["task_layer"] == layer)[0] if g["task_mode"][t] != 2]
        assert sum(r["n"] for r in rows) == len(real)
        assert [r["start"] for r in rows] == sorted(r["start"] for r in rows)
        assert rows[0]["gap"] is None and rows[0]["start"] == 0.0
        for a, b in zip(rows, rows[1:]):
            assert abs(b["gap"] - (b["start"] - a["end"])) < 1e-9
        assert all(r["span"] >= r["task"] - 1e-9 for r in rows)
    text = trace_phases.markdown(trace_phases.phase_table(rec, TICKS_PER_UNIT, g, 0))
    assert text.count("\n") == 1 + len(trace_phases.phase_table(rec, TICKS_PER_UNIT, g, 0))
