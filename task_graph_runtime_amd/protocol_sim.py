"""CPU model of the in-kernel runtime protocol, run on an exported tGraph.

The persistent kernel's workers and schedulers (MPK summary page, section 2
Q2: workers pop FIFO task queues, schedulers consume event queues; section 4
"6 minimum checks": a task waits on one event whose counter must reach its
trigger count, the consumers of an event form a contiguous range) are
simulated as agents whose every memory operation happens at a random time,
so that many interleavings of one step -- and of several steps in a row on
the same never-reset counters -- can be explored on the host:

* a worker holds its next ahead-of-time (AOT) task; while that task's
  dependent event has not reached counts * epoch it serves its just-in-time
  (JIT) ring; with no AOT task left it serves the ring until the end event
  fires;
* a finished task arrives at its triggering event: a sole e' event (one
  producer, only empty consumers) fires without a counter; an event with at
  least TWO_LEVEL_MIN producers counts on SUB sub-counters first (producer t
  on sub-counter t mod SUB, the arrival that completes a sub-counter's quota
  adds 1 to the event counter, which fires at (non-empty sub-counters) *
  epoch); any other event fires at counts * epoch;
* the agent whose arrival fires an event resolves its empty consumers on the
  spot, each empty arriving at its own event, one level of cascade (a graph
  built without fusion has fan-out empties feeding fan-in empties), and
  hands an event with JIT consumers to the schedulers: its tasks take
  consecutive worker positions from the running count of JIT tasks in event
  order (mod W), one ring entry per scheduler segment the positions cross,
  segment c going to scheduler (P_e / n_sub + c) mod S, which writes each
  task into the ring of the worker at its position (position p is worker
  p // n_sub + S * (p mod n_sub));
* everything exits when the end event fires.

`simulate` checks, for every step: termination (no agent waits forever), that
every non-empty task runs exactly once and every empty task is resolved
exactly once, that a task starts only after every task it transitively waits
for (through events and empty tasks) has finished, and after the last step
that every counter equals its per-step target times the number of steps.  A
violated check raises ProtocolError.

The model follows the protocol as the runtime implements it (the two-level
threshold, sub-counter rule, sole events and JIT positions above are the
runtime's); it is not the device code and shares no code with it.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field

import numpy as np

MODE_AOT, MODE_JIT, MODE_EMPTY = 0, 1, 2
HAS_JIT, HAS_EMPTY = 1, 2
SUB = 8
TWO_LEVEL_MIN = 64


class ProtocolError(AssertionError):
    pass


@dataclass
class SimStats:
    steps: int = 0
    actions: int = 0
    polls: int = 0
    jit_tasks: int = 0
    max_ring: int = 0
    makespan: list = field(default_factory=list)
    # the last step's schedule in the layout of TGraph.read_trace (times in
    # TICKS_PER_UNIT ticks per simulated time unit), when simulate(trace=True)
    trace: object = None


TICKS_PER_UNIT = 100.0
TRACE_DTYPE = np.dtype([("task", np.int32), ("worker", np.int32), ("t_wait", np.uint64), ("t_start", np.uint64),
                        ("t_end", np.uint64), ("t_done", np.uint64), ("t_mark", np.uint64, (2,))])


def _predecessors(g: dict) -> list:
    """For every task, the set of non-empty tasks it waits for directly:
    the producers of its dependent event, looking through empty producers
    (an empty task's producers are those of its own dependent event)."""
    NT = len(g["task_type"])
    trig, dep, mode = g["task_trig"], g["task_dep"], g["task_mode"]
    prod = [[] for _ in range(len(g["event_counts"]))]
    for t in range(NT):
        if trig[t] >= 0:
            prod[trig[t]].append(t)
    memo = {}

    def real_producers(e):
        if e in memo:
            return memo[e]
        out = set()
        for p in prod[e]:
            if mode[p] == MODE_EMPTY:
                out |= real_producers(int(dep[p]))
            else:
                out.add(p)
        memo[e] = out
        return out

    return [real_producers(int(dep[t])) if dep[t] >= 0 else set() for t in range(NT)]


def simulate(g: dict, steps: int = 2, seed: int = 0, task_time=(1.0, 20.0), op_time=(0.05, 3.0),
             must_follow=None, trace: bool = False) -> SimStats:
    """Run `steps` steps of the runtime protocol on graph `g` (the dict of
    ``TGraph.export()``), with task durations uniform in `task_time` and
    every memory operation (poll, arrival, ring write) delayed uniformly in
    `op_time`.  A waiting agent is woken (after such a delay) when a counter
    it polls changes or its ring receives an entry, which is when one of its
    polls could first succeed; an agent left waiting when nothing else can
    happen is a deadlock.  `must_follow[t]`, when given, lists the tasks
    (linear indices) that must have finished when task t starts -- a relation
    taken from somewhere other than the graph's own events, such as the
    overlap of the tasks' regions; by default the graph's events define it.
    With `trace`, the statistics carry the last step's schedule as trace
    records (trace_export renders them like a device trace).  Returns
    statistics; raises ProtocolError on a violated check."""
    rng = np.random.default_rng(seed)
    ttype, mode = np.asarray(g["task_type"]), np.asarray(g["task_mode"])
    dep, trig = np.asarray(g["task_dep"], np.int64), np.asarray(g["task_trig"], np.int64)
    counts = np.asarray(g["event_counts"], np.int64)
    first, last = np.asarray(g["event_first"], np.int64), np.asarray(g["event_last"], np.int64)
    flags = np.asarray(g["event_flags"], np.int64)
    hdr, prm = g["header"], g["params"]
    NT, NE = len(ttype), len(counts)
    W = int(prm["n_workers"])
    S = int(prm["n_sched_waves"])
    end_ev = int(hdr["end"])
    aot_off, aot_tasks = np.asarray(g["aot_offsets"], np.int64), np.asarray(g["aot_tasks"], np.int64)
    preds = _predecessors(g) if must_follow is None else [set(int(x) for x in m) for m in must_follow]

    # per-event device records, as the runtime sets them up
    quota = np.zeros((NE, SUB), np.int64)
    for t in range(NT):
        if trig[t] >= 0:
            quota[trig[t], t % SUB] += 1
    two_level = counts >= TWO_LEVEL_MIN
    dev_counts = np.where(two_level, (quota > 0).sum(axis=1), counts)
    sole = np.zeros(NE, bool)
    for e in range(NE):
        if counts[e] == 1 and last[e] >= first[e]:
            sole[e] = bool(np.all(mode[first[e]:last[e] + 1] == MODE_EMPTY))
        # the firing agent resolves every consumer of an event with empty
        # consumers as an empty task: such an event must have no other kind
        if (flags[e] & HAS_EMPTY) and not np.all(mode[first[e]:last[e] + 1] == MODE_EMPTY):
            raise ProtocolError(f"event {e} has empty and non-empty consumers")
    has_jit = (flags & HAS_JIT) != 0
    if has_jit.any() and S < 1:
        raise ProtocolError("graph has JIT tasks but no schedulers")
    n_sub = W // max(1, S)
    start_pos = np.zeros(NE, np.int64)
    pos = 0
    for e in range(NE):
        if has_jit[e]:
            start_pos[e] = pos % W
            pos += last[e] - first[e] + 1

    ev_cnt = np.zeros(NE, np.int64)
    ev_sub = np.zeros((NE, SUB), np.int64)
    sched_ring = [[] for _ in range(max(1, S))]      # entries (event, chunk)
    sched_head = [0] * max(1, S)
    jit_ring = [[] for _ in range(W)]                # task ids
    jit_head = [0] * W
    stats = SimStats()

    def u(lo_hi):
        return float(rng.uniform(*lo_hi))

    for step in range(1, steps + 1):
        epoch = step
        runs = np.zeros(NT, np.int64)
        t_start = np.full(NT, np.nan)
        t_end = np.full(NT, np.nan)
        t_wait = np.full(NT, np.nan)
        ran_on = np.full(NT, -1, np.int64)
        idle_since = [0.0] * W
        # agents: ("w", w) and ("s", s); per-worker AOT cursor
        cursor = [int(aot_off[w]) for w in range(W)]
        q = []
        seq = [0]

        def push(time, kind, idx, payload=None):
            seq[0] += 1
            heapq.heappush(q, (time, seq[0], kind, idx, payload))

        waiters = {}            # event -> workers whose next AOT task (or exit) waits on its counter

        def wake_all(e, now):
            for w in waiters.pop(e, ()):
                push(now + u(op_time), "w", w)

        def arrive(e, task, now):
            """One arrival at event e by `task`; True when it fires e."""
            if sole[e]:
                return True
            if two_level[e]:
                k = task % SUB
                ev_sub[e, k] += 1
                if ev_sub[e, k] != quota[e, k] * epoch:
                    return False
            ev_cnt[e] += 1
            wake_all(e, now)
            return ev_cnt[e] == dev_counts[e] * epoch

        def hand_over(e, now):
            k = int(last[e] - first[e] + 1)
            P = int(start_pos[e])
            n_ch = (P + k - 1) // n_sub - P // n_sub + 1
            for c in range(n_ch):
                s = (P // n_sub + c) % S
                sched_ring[s].append((e, c))
                push(now + u(op_time), "s", s)          # wake the scheduler

        def fire(e, now):
            """Event e has fired at `now` (by the arriving agent)."""
            if flags[e] & HAS_EMPTY:
                for t in range(int(first[e]), int(last[e]) + 1):
                    if mode[t] != MODE_EMPTY:
                        continue
                    runs[t] += 1
                    t_start[t] = t_end[t] = now
                    f = int(trig[t])
                    if arrive(f, t, now):
                        if has_jit[f]:
                            hand_over(f, now)
                        if flags[f] & HAS_EMPTY:      # one level of cascade
                            for t2 in range(int(first[f]), int(last[f]) + 1):
                                if mode[t2] != MODE_EMPTY:
                                    continue
                                runs[t2] += 1
                                t_start[t2] = t_end[t2] = now
                                f2 = int(trig[t2])
                                if arrive(f2, t2, now):
                                    if has_jit[f2]:
                                        hand_over(f2, now)
                                    if flags[f2] & HAS_EMPTY:
                                        raise ProtocolError(f"empty chain deeper than two at event {f2}")
            if has_jit[e]:
                hand_over(e, now)
            if e == end_ev:
                for s in range(S):
                    push(now + u(op_time), "s", s)

        def start_task(task, w, now):
            if mode[task] == MODE_EMPTY:
                raise ProtocolError(f"worker {w} was handed empty task {task}")
            for p in preds[task]:
                if not (t_end[p] <= now):
                    raise ProtocolError(f"step {step}: task {task} started at {now:.2f} before its producer {p} "
                                        f"finished ({t_end[p]})")
            runs[task] += 1
            t_start[task] = now
            t_wait[task] = idle_since[w]
            ran_on[task] = w
            dur = u(task_time)
            push(now + dur, "end", w, task)

        # the root event's consumers need no arrival (counts 0); launch all agents
        for w in range(W):
            push(u(op_time), "w", w)
        for s in range(S):
            push(u(op_time), "s", s)
        running = [None] * W
        alive_w, alive_s = set(range(W)), set(range(S))
        now = 0.0
        while q:
            now, _, kind, idx, payload = heapq.heappop(q)
            stats.actions += 1
            if kind == "end":          # task `payload` of worker idx finishes, then triggers
                task = int(payload)
                t_end[task] = now
                idle_since[idx] = now
                running[idx] = None
                e = int(trig[task])
                if arrive(e, task, now):
                    fire(e, now)
                push(now + u(op_time), "w", idx)
                continue
            if kind == "w":
                w = idx
                if w not in alive_w or running[w] is not None:
                    continue
                stats.polls += 1
                # one poll: the JIT slot, the next AOT task's counter (or the end event's) and act
                if jit_head[w] < len(jit_ring[w]):
                    task = jit_ring[w][jit_head[w]]
                    jit_head[w] += 1
                    stats.jit_tasks += 1
                    running[w] = task
                    start_task(task, w, now)
                    continue
                if cursor[w] < aot_off[w + 1]:
                    task = int(aot_tasks[cursor[w]])
                    e = int(dep[task])
                    target = dev_counts[e] * epoch
                    if ev_cnt[e] >= target:
                        cursor[w] += 1
                        running[w] = task
                        start_task(task, w, now)
                        continue
                    waiters.setdefault(e, set()).add(w)
                elif ev_cnt[end_ev] >= dev_counts[end_ev] * epoch:
                    alive_w.discard(w)
                else:
                    waiters.setdefault(end_ev, set()).add(w)
                continue
            if kind == "s":
                s = idx
                if s not in alive_s:
                    continue
                if sched_head[s] < len(sched_ring[s]):
                    e, c = sched_ring[s][sched_head[s]]
                    sched_head[s] += 1
                    P = int(start_pos[e])
                    k = int(last[e] - first[e] + 1)
                    seg = P // n_sub + c
                    u0, u1 = max(P, seg * n_sub), min(P + k, (seg + 1) * n_sub)
                    for uu in range(u0, u1):
                        lane = uu - seg * n_sub
                        w = s + lane * S
                        task = int(first[e] + (uu - P))
                        jit_ring[w].append(task)
                        stats.max_ring = max(stats.max_ring, len(jit_ring[w]) - jit_head[w])
                        push(now + u(op_time), "w", w)
                    push(now + u(op_time), "s", s)
                    continue
                if ev_cnt[end_ev] >= dev_counts[end_ev] * epoch:
                    alive_s.discard(s)
                continue
        if alive_w or alive_s:
            raise ProtocolError(f"step {step}: agents left waiting: workers {sorted(alive_w)[:8]}, "
                                f"schedulers {sorted(alive_s)[:8]}")
        bad = np.nonzero(runs != 1)[0]
        if len(bad):
            t = int(bad[0])
            raise ProtocolError(f"step {step}: task {t} (type {int(ttype[t])}, mode {int(mode[t])}) ran {int(runs[t])} times")
        for w in range(W):
            if jit_head[w] != len(jit_ring[w]):
                raise ProtocolError(f"step {step}: worker {w} left {len(jit_ring[w]) - jit_head[w]} JIT tasks unserved")
        for s in range(S):
            if sched_head[s] != len(sched_ring[s]):
                raise ProtocolError(f"step {step}: scheduler {s} left ring entries unserved")
        stats.makespan.append(float(np.nanmax(t_end)))
        stats.steps = step
        if trace and step == steps:
            done = np.nonzero(ran_on >= 0)[0]
            rec = np.zeros(len(done), TRACE_DTYPE)
            rec["task"] = done
            rec["worker"] = ran_on[done]
            for k, v in (("t_wait", t_wait), ("t_start", t_start), ("t_end", t_end), ("t_done", t_end)):
                rec[k] = np.round(v[done] * TICKS_PER_UNIT).astype(np.uint64)
            stats.trace = rec

    # counters after `steps` steps: never reset, each at its per-step target times the steps
    for e in range(NE):
        if sole[e]:
            want_main = 0
        else:
            want_main = dev_counts[e] * steps
        if ev_cnt[e] != want_main:
            raise ProtocolError(f"event {e}: counter {ev_cnt[e]} after {steps} steps, expected {want_main}")
        if two_level[e] and not np.array_equal(ev_sub[e], quota[e] * steps):
            raise ProtocolError(f"event {e}: sub-counters {ev_sub[e].tolist()} after {steps} steps")
    return stats
