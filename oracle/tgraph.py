"""tGraph oracle: the canonical task/event-graph spec (v1) and a brute-force checker.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Plain Python/numpy; it
shares no code with the C++ builder and is compared with it bit for bit.

What the pages fix (MPK summary page, "MPK: A Compiler and Runtime for
Mega-Kernelizing Tensor Programs -- L2"):

* section 2 (Q2, the method): operators are decomposed into per-tile tasks;
  an event links two tasks iff the producer's output region overlaps the
  consumer's input region; the graph is then fused, normalised and
  linearised into a compact device structure;
* section 4, "Successor-set fusion (Def 4.1)" and "Predecessor-set fusion
  (Def 4.2)": events with equal consumer sets, then equal producer sets, merge;
* section 4, "6 minimum checks" (check 3) and section 7 ("Empty tasks as
  degree-reduction glue"): normalisation adds one event e' and k empty tasks
  per fan-out (and, for a graph built without fusion, per fan-in) so that
  every task has <= 1 dependent and <= 1 triggering event;
* section 4 check 4 (Alg 1): BFS linearisation places the dependent tasks of
  each dequeued event consecutively, so fan-out is a ``[first, last]`` range;
* section 4, design-space table: JIT for data-dependent attention, AOT for
  the rest.  Which attention counts as data-dependent is a parameter
  (``Params.jit_attn``); the library's default makes it JIT at batch > 1,
  where an event's splits serve requests of different lengths, and AOT at
  batch 1, where every split of the step has the same pages.  The two ends
  of the design space, every task AOT and every task JIT
  (``Params.jit_all``), are the scheduling ablation.
The HN comment (item 2) fixes the dependency rule: B depends on A iff A
produces any element B consumes.

Where the pages leave a step open the plainest reading is taken (order of
Def 4.1 then Def 4.2; Kahn-style BFS that enqueues an event when its last
producer is placed; a root event for sources and an end event for sinks;
``counts(e) = |InTasks(e)|``; empty tasks numbered after the originals;
round-robin AOT placement in linear order).  Balanced tiling: an operator
with ``N`` output columns is cut, on a quantum of ``q`` columns, into ``T``
tiles ``[q*floor(n*U/T), min(N, q*floor((n+1)*U/T)))`` with ``U = ceil(N/q)``.
The fused q/k/v projection writes its columns group-major -- for kv group
``g``: its ``G`` query heads, then its key head, then its value head -- and
is tiled within each group (``T_qkv / n_kv_heads`` tiles per group), so each
attention split reads one contiguous column block produced by the tiles of
its own group and no projection tile feeds two groups.

K-split (batch > 1, a choice of this build): the q/k/v, O and down
projections cut their input dimension into ``K_qkv``, ``K_o``, ``K_down``
ranges (on a quantum of 32), and tile ``n`` of a projection is column tile
``n // K`` over k-range ``n % K``.  Each k-range writes its own plane of
partial sums (``[plane][b][column]``), and every reader of those outputs
(attention splits, norm tasks) adds the planes.  A tile then reads only its
k-range of the activations, which at batch 16 are as many bytes as the
weights of a 16-row tile.  At batch 1 every K is 1.

Operator fusion (a choice of this build, not of the pages; the rewrites
below apply unchanged to whatever tasks the decomposition emits): q/k
RMSNorm + RoPE, the KV-cache append and the split combine run inside the
attention tasks, and at batch 1 the residual add + RMSNorm run inside the
projection tiles that consume them (``fused_norm``).  Type ids 3
(QKNORM_ROPE) and 5 (COMBINE) are therefore never emitted for the decoder.

Attention slots (a choice of this build): kv group ``g`` has ``M = S_attn``
attention tasks, task ``(j, g)`` being slot ``j`` of the group (at batch 1
the slots are the request's splits).  Which request a slot serves is decided
when the step runs, from the sequence lengths, so that every slot gets
about the same number of pages (a request with more cached tokens gets more
splits); ``M >= B`` gives every request at least one.  A slot may therefore
serve any request of its group, and every attention task declares the whole
group: all B rows of the group's q/k/v columns as input; the group's partial
records, attention output and cache rows of all B requests as outputs.  The
events are the same as with per-request boxes (the group's projection tiles
cover all B rows, and the O projection reads every group).
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass

import numpy as np

# task types (3 and 5 are kept as ids for the generic entry; the decoder emits neither)
EMBED, ATTN_NORM, QKV, QKNORM_ROPE, ATTN, COMBINE, OPROJ, MLP_NORM, GATEUP, DOWN, FINAL_NORM, LMHEAD, ARGMAX, \
    EMPTY, ROUTER, EXPERT_GU, EXPERT_DOWN = range(17)
TYPE_NAMES = ["EMBED", "ATTN_NORM", "QKV", "QKNORM_ROPE", "ATTN", "COMBINE", "OPROJ", "MLP_NORM", "GATEUP", "DOWN",
              "FINAL_NORM", "LMHEAD", "ARGMAX", "EMPTY", "ROUTER", "EXPERT_GU", "EXPERT_DOWN"]
# tasks whose work is decided by data when the step runs (the attention's
# splits, the experts a slot serves): JIT under the hybrid policy
DATA_DEPENDENT = (ATTN, EXPERT_GU, EXPERT_DOWN)
MODE_AOT, MODE_JIT, MODE_EMPTY = 0, 1, 2
FLAG_HAS_JIT, FLAG_HAS_EMPTY = 1, 2

# tensors: five shared ones, then 15 per layer (rlog and route in mixture-of-experts layers)
T_E, T_HF, T_LOGITS, T_PMAX, T_NEXT = range(5)
L_R, L_H, L_QKV, L_Q, L_KC, L_VC, L_PART, L_ATTN, L_O, L_S, L_H2, L_A, L_D, L_RLOG, L_ROUTE = range(15)
N_LAYER_TENSORS = 15


def layer_tensor(l, k):
    return 5 + N_LAYER_TENSORS * l + k


@dataclass
class Params:
    W: int                # worker count
    S_sched: int = 16     # scheduler wavefronts
    q: int = 1            # column quantum of GEMV tiles
    T_qkv: int = 1
    T_o: int = 1
    T_gu: int = 1
    T_down: int = 1
    T_lm: int = 1
    S_attn: int = 1
    jit_attn: bool = True   # attention tasks JIT (else AOT)
    jit_all: bool = False   # every non-empty task JIT
    coarse: bool = False    # operator-level graph: every task waits for the whole previous operator
    K_qkv: int = 1          # k-splits of the q/k/v, O and down projections (batch > 1)
    K_o: int = 1
    K_down: int = 1
    fusion: int = 0         # 0: Def 4.1 then Def 4.2; 1: no fusion (one event per overlap edge)
    T_router: int = 1       # mixture of experts: router tiles, gate/up and down tiles per expert slot
    T_egu: int = 1
    T_edown: int = 1


def tile_range(N, q, T, n):
    U = -(-N // q)
    return q * (n * U // T), min(N, q * ((n + 1) * U // T))


def _box(tensor, lo, hi):
    lo = tuple(lo) + (0,) * (4 - len(lo))
    hi = tuple(hi) + (1,) * (4 - len(hi))
    return (tensor, lo, hi)


def fused_norm(B):
    """Whether RMSNorm runs inside the projection tiles that consume it.

    At batch 1 every projection tile stages its whole input vector on chip, so
    the residual add and RMSNorm are recomputed by each consuming tile (a
    prologue) instead of running as a task of their own; the first tile of
    the consuming projection also stores the residual for later layers.  At
    batch > 1 the norms stay tasks (ATTN_NORM, MLP_NORM, FINAL_NORM) and the
    embedding EMBED tasks, one task per request: coords (b,), output row b.
    A norm task declares all B rows of its inputs, though it reads row b
    only: every norm task of an operator then has the same producer set and
    the B tasks share one event, instead of B events that every producer
    tile would have to trigger (B rewrites per tile).
    """
    return B == 1


def decompose(cfg, B, P, prm: Params):
    """Operators -> tasks with their input/output boxes, in program order.

    Returns a list of dicts ``{type, layer, coords, ins, outs}``; a box is
    ``(tensor_id, lo[4], hi[4])`` (half-open).

    Per layer: [ATTN_NORM] QKV tiles, ATTN(j, g) [JIT], OPROJ tiles,
    [MLP_NORM] GATEUP tiles, DOWN tiles; then [FINAL_NORM] LMHEAD tiles and
    ARGMAX (bracketed tasks only at batch > 1, see ``fused_norm``).  An
    attention split also applies q/k RMSNorm and RoPE to its query heads, the
    last split of a request appends the new key/value to the cache, and the
    last split of a request to finish merges the request's partials into the
    attention output (attention tasks declare their whole kv group, see the
    module docstring on slots).
    """
    L = cfg["n_layers"]; H = cfg["hidden"]; hq = cfg["n_q_heads"]; hkv = cfg["n_kv_heads"]; d = cfg["head_dim"]
    F = cfg["ffn"]; V = cfg["vocab"]; S = prm.S_attn
    G = hq // hkv
    Sg = (G + 2) * d          # qkv columns of one kv group: G q heads, then k, then v
    maxs = cfg["max_seq_len"]
    fused = fused_norm(B)
    tasks = []

    def add(tp, layer, coords, ins, outs):
        c = tuple(coords) + (0,) * (3 - len(coords))
        tasks.append(dict(type=tp, layer=layer, coords=c, ins=ins, outs=outs))

    full = lambda tn, n: _box(tn, (0, 0), (B, n))
    row = lambda tn, b, n: _box(tn, (b, 0), (b + 1, n))
    # q/k/v, O and down outputs have one plane of partial sums per k-split:
    # [plane][b][column]; their readers take all planes
    planes = lambda tn, ks, n: _box(tn, (0, 0, 0), (ks, B, n))
    Kq, Ko, Kd = prm.K_qkv, prm.K_o, prm.K_down
    E, Kx, Fe = cfg.get("n_experts", 0), cfg.get("top_k", 0), cfg.get("moe_ffn", 0)
    moe = E > 0
    M = min(E, B * Kx)        # expert slots of a layer: the distinct experts the batch chose, at most

    def moe_layer(l, t, mid):
        """The mixture-of-experts FFN of layer l (MPK summary section 5, Fig 10):
        ROUTER tiles (router logits; at batch 1 they also normalise, and tile
        0 stores the residual s_l and the normalised h2_l the experts read),
        then per
        expert slot s (the s-th distinct expert the batch chose, decided when
        the step runs) EXPERT_GU tiles (tile 0 also writes the slot's route
        record: expert, tokens, weights) and EXPERT_DOWN tiles, which add
        their tokens' weighted outputs into d_l.  A slot's down tiles read only
        its route record and its gate/up output, so they wait for that slot
        alone.  d_l starts the step at zero: the task that stores s_l (router
        tile 0 at batch 1, MLP_NORM b at batch > 1, row b) zeroes it, with the
        same readers as s_l, so the zeroing adds no event."""
        for n in range(prm.T_router):
            elo, ehi = tile_range(E, prm.q, prm.T_router, n)
            outs = [_box(t(L_RLOG), (0, elo), (B, ehi))]
            if fused and n == 0:
                outs += [full(t(L_S), H), full(t(L_H2), H), planes(t(L_D), 1, H)]
            add(ROUTER, l, (n,), mid if fused else [full(t(L_H2), H)], outs)
        rec = 2 + 2 * B
        for s_ in range(M):
            for n in range(prm.T_egu):
                lo, hi = tile_range(Fe, prm.q, prm.T_egu, n)
                outs = [_box(t(L_A), (s_, 0, lo), (s_ + 1, B, hi))]
                if n == 0:
                    outs.append(_box(t(L_ROUTE), (s_, 0), (s_ + 1, rec)))
                add(EXPERT_GU, l, (s_, n), [full(t(L_RLOG), E), full(t(L_H2), H)], outs)
        for s_ in range(M):
            for n in range(prm.T_edown):
                lo, hi = tile_range(H, prm.q, prm.T_edown, n)
                add(EXPERT_DOWN, l, (s_, n), [_box(t(L_ROUTE), (s_, 0), (s_ + 1, rec)),
                                              _box(t(L_A), (s_, 0, 0), (s_ + 1, B, Fe))],
                    [_box(t(L_D), (0, 0, lo), (1, B, hi))])

    if not fused:
        for b in range(B):
            add(EMBED, -1, (b,), [], [row(T_E, b, H)])
    for l in range(L):
        t = lambda k: layer_tensor(l, k)
        prev = [] if l == 0 else [full(layer_tensor(l - 1, L_S), H), planes(layer_tensor(l - 1, L_D), Kd, H)]
        if not fused:
            for b in range(B):
                add(ATTN_NORM, l, (b,), prev if l else [full(T_E, H)], [row(t(L_R), b, H), row(t(L_H), b, H)])
        tpg = prm.T_qkv // hkv
        for n in range(prm.T_qkv):
            g, r = divmod(n, tpg)
            j, ks = divmod(r, Kq)
            lo, hi = tile_range(Sg, prm.q, tpg // Kq, j)
            klo, khi = tile_range(H, 32, Kq, ks)
            outs = [_box(t(L_QKV), (ks, 0, g * Sg + lo), (ks + 1, B, g * Sg + hi))]
            if fused and n == 0:
                outs.append(full(t(L_R), H))
            # (coarse: the operator-level graph of the pages' ablation, where a task
            # waits for the whole previous operator, so a k-split tile declares its
            # whole input row)
            add(QKV, l, (n,), prev if fused else [full(t(L_H), H) if prm.coarse else _box(t(L_H), (0, klo), (B, khi))],
                outs)
        for g in range(hkv):
            for j in range(S):
                outs = [_box(t(L_PART), (0, g, 0, 0), (1, g + 1, S, G * (d + 2))),
                        _box(t(L_ATTN), (0, g * G * d), (B, (g + 1) * G * d)),
                        _box(t(L_KC), (0, 0, g, 0), (B, maxs, g + 1, d)),
                        _box(t(L_VC), (0, 0, g, 0), (B, maxs, g + 1, d))]
                qin = (_box(t(L_QKV), (0, 0, 0), (Kq, B, hkv * Sg)) if prm.coarse
                       else _box(t(L_QKV), (0, 0, g * Sg), (Kq, B, (g + 1) * Sg)))
                add(ATTN, l, (j, g), [qin], outs)
        for n in range(prm.T_o):
            c, ks = divmod(n, Ko)
            lo, hi = tile_range(H, prm.q, prm.T_o // Ko, c)
            klo, khi = tile_range(hq * d, 32, Ko, ks)
            oin = full(t(L_ATTN), hq * d) if prm.coarse else _box(t(L_ATTN), (0, klo), (B, khi))
            add(OPROJ, l, (n,), [oin], [_box(t(L_O), (ks, 0, lo), (ks + 1, B, hi))])
        mid = [full(t(L_R), H), planes(t(L_O), Ko, H)]
        if not fused:
            for b in range(B):
                add(MLP_NORM, l, (b,), mid, [row(t(L_S), b, H), row(t(L_H2), b, H)]
                    + ([_box(t(L_D), (0, b, 0), (1, b + 1, H))] if moe else []))
        if moe:
            moe_layer(l, t, mid)
            continue
        for n in range(prm.T_gu):
            lo, hi = tile_range(F, prm.q, prm.T_gu, n)
            outs = [_box(t(L_A), (0, lo), (B, hi))]
            if fused and n == 0:
                outs.append(full(t(L_S), H))
            add(GATEUP, l, (n,), mid if fused else [full(t(L_H2), H)], outs)
        for n in range(prm.T_down):
            c, ks = divmod(n, Kd)
            lo, hi = tile_range(H, prm.q, prm.T_down // Kd, c)
            klo, khi = tile_range(F, 32, Kd, ks)
            din = full(t(L_A), F) if prm.coarse else _box(t(L_A), (0, klo), (B, khi))
            add(DOWN, l, (n,), [din], [_box(t(L_D), (ks, 0, lo), (ks + 1, B, hi))])
    last = [full(layer_tensor(L - 1, L_S), H), planes(layer_tensor(L - 1, L_D), Kd, H)]
    if not fused:
        for b in range(B):
            add(FINAL_NORM, -1, (b,), last, [row(T_HF, b, H)])
    for n in range(prm.T_lm):
        lo, hi = tile_range(V, prm.q, prm.T_lm, n)
        add(LMHEAD, -1, (n,), last if fused else [full(T_HF, H)],
            [_box(T_LOGITS, (0, lo), (B, hi)), _box(T_PMAX, (0, n, 0), (B, n + 1, 2))])
    add(ARGMAX, -1, (), [_box(T_PMAX, (0, 0, 0), (B, prm.T_lm, 2))], [_box(T_NEXT, (0,), (B,))])
    return tasks


def producer_sets(tasks):
    """Brute-force overlap dependencies: ``P[c]`` = producers ``p < c`` whose
    output box meets an input box of ``c`` on the same tensor (all dims)."""
    outs, ins = {}, {}
    for i, t in enumerate(tasks):
        for (tn, lo, hi) in t["outs"]:
            outs.setdefault(tn, []).append((i, lo, hi))
        for (tn, lo, hi) in t["ins"]:
            ins.setdefault(tn, []).append((i, lo, hi))
    P = [set() for _ in tasks]
    for tn, il in ins.items():
        ol = outs.get(tn)
        if not ol:
            continue
        ot = np.array([x[0] for x in ol]); olo = np.array([x[1] for x in ol]); ohi = np.array([x[2] for x in ol])
        it = np.array([x[0] for x in il]); ilo = np.array([x[1] for x in il]); ihi = np.array([x[2] for x in il])
        ov = np.all((olo[:, None, :] < ihi[None, :, :]) & (ilo[None, :, :] < ohi[:, None, :]), axis=2)
        ov &= ot[:, None] < it[None, :]
        pi, ci = np.nonzero(ov)
        for a, b in zip(ot[pi], it[ci]):
            P[int(b)].add(int(a))
    return P


FUSION_A, FUSION_OFF = 0, 1


def canonicalize(tasks, W, jit_attn=True, jit_all=False, fusion=FUSION_A):
    """Fusion (Def 4.1 then 4.2, or none), normalisation, Kahn-BFS
    linearisation, classification and AOT placement.  Returns the exported
    arrays (dict).

    ``fusion=FUSION_OFF`` keeps one event per overlap edge ``(p, c)``
    (In = {p}, Out = {c}, pre-ordered by ``(c, p)``); a consumer then depends
    on several events and normalisation needs the fan-in rewrite besides the
    fan-out one (MPK summary section 4, "6 minimum checks", check 3)."""
    N = len(tasks)
    P = producer_sets(tasks)

    if fusion == FUSION_A:
        # Def 4.1: one event per consumer with all its producers; Def 4.2: merge equal producer sets.
        groups = {}
        for c in range(N):
            if P[c]:
                groups.setdefault(frozenset(P[c]), []).append(c)
        fused = sorted(([sorted(k), sorted(v)] for k, v in groups.items()), key=lambda e: min(e[1]))
        # fixpoint: Out-sets disjoint, In-sets distinct
        seen_out = set()
        for _, o in fused:
            assert not (seen_out & set(o))
            seen_out |= set(o)
        assert len({tuple(i) for i, _ in fused}) == len(fused)
    elif fusion == FUSION_OFF:
        fused = [[[p], [c]] for c in range(N) for p in sorted(P[c])]
    else:
        raise ValueError("fusion must be FUSION_A or FUSION_OFF")

    ev_in = [list(i) for i, _ in fused]
    ev_out = [list(o) for _, o in fused]
    deps_of = [[] for _ in range(N)]
    for e, o in enumerate(ev_out):
        for c in o:
            deps_of[c].append(e)         # in pre-order
    trigs_of = [[] for _ in range(N)]
    for e, i in enumerate(ev_in):
        for p in i:
            trigs_of[p].append(e)        # in pre-order

    # normalisation, task by task in original order: a task with k >= 2
    # dependent events (fan-in, only without fusion) gets a new event e' that
    # k empty tasks trigger, empty i waiting on the i-th event; a task with
    # k >= 2 triggering events (fan-out) gets a new event e' that k empty
    # tasks wait on, empty i triggering the i-th event.  Empty tasks are
    # numbered after the originals in the order they are made; coords (i, 0)
    # for a fan-out empty, (i, 1) for a fan-in one.
    ttype = [t["type"] for t in tasks]
    tlayer = [t["layer"] for t in tasks]
    tcoords = [t["coords"] for t in tasks]
    torig = list(range(N))
    n_empty = 0
    dep = {}
    trig = {}

    def new_empty(t, i, kind):
        nonlocal n_empty
        T = len(ttype)
        ttype.append(EMPTY); tlayer.append(tlayer[t]); tcoords.append((i, kind, 0))
        torig.append(-1 - n_empty); n_empty += 1
        return T

    for t in range(N):
        dl = deps_of[t]
        if len(dl) >= 2:
            ep = len(ev_in)
            ev_in.append([]); ev_out.append([t])
            for i, e in enumerate(dl):
                T = new_empty(t, i, 1)
                dep[T] = e; trig[T] = ep
                ev_in[ep].append(T)
                ev_out[e] = [T if x == t else x for x in ev_out[e]]
            dep[t] = ep
        elif len(dl) == 1:
            dep[t] = dl[0]
        tr = trigs_of[t]
        if len(tr) >= 2:
            ep = len(ev_in)
            ev_in.append([t]); ev_out.append([])
            for i, e in enumerate(tr):
                T = new_empty(t, i, 0)
                dep[T] = ep; trig[T] = e
                ev_out[ep].append(T)
                ev_in[e] = [T if x == t else x for x in ev_in[e]]
            trig[t] = ep
        elif len(tr) == 1:
            trig[t] = tr[0]
    NT = len(ttype)
    root = len(ev_in); ev_in.append([]); ev_out.append([])
    end = len(ev_in); ev_in.append([]); ev_out.append([])
    for t in range(NT):
        if t not in dep:
            dep[t] = root; ev_out[root].append(t)
        if t not in trig:
            trig[t] = end; ev_in[end].append(t)
    NE = len(ev_in)
    counts = [len(x) for x in ev_in]

    # Kahn-BFS linearisation
    indeg = list(counts)
    new_ev = [-1] * NE; new_task = [-1] * NT
    first = [0] * NE; last = [0] * NE
    q = deque([root]); ne = 0; nt = 0
    while q:
        e = q.popleft()
        new_ev[e] = ne; ne += 1
        first[e] = nt
        for t in sorted(ev_out[e]):
            new_task[t] = nt; nt += 1
            f = trig[t]
            indeg[f] -= 1
            if indeg[f] == 0:
                q.append(f)
        last[e] = nt - 1
    if nt != NT:
        raise ValueError("tGraph has a cycle")

    order = sorted(range(NT), key=lambda t: new_task[t])
    eorder = sorted(range(NE), key=lambda e: new_ev[e])
    # JIT tasks are handed over when their event fires; the root event is
    # never triggered, so its consumers stay AOT under every policy
    mode = {EMPTY: MODE_EMPTY}
    mode.update({ty: MODE_JIT if jit_attn or jit_all else MODE_AOT for ty in DATA_DEPENDENT})
    other = MODE_JIT if jit_all else MODE_AOT

    def mode_of(t):
        m = mode.get(ttype[t], other)
        return MODE_AOT if m == MODE_JIT and dep[t] == root else m

    out = {
        "task_type": np.array([ttype[t] for t in order], dtype=np.uint8),
        "task_mode": np.array([mode_of(t) for t in order], dtype=np.uint8),
        "task_layer": np.array([tlayer[t] for t in order], dtype=np.int16),
        "task_coords": np.array([tcoords[t] for t in order], dtype=np.uint16).reshape(NT, 3),
        "task_orig": np.array([torig[t] for t in order], dtype=np.int32),
        "task_dep": np.array([new_ev[dep[t]] for t in order], dtype=np.int32),
        "task_trig": np.array([new_ev[trig[t]] for t in order], dtype=np.int32),
        "event_counts": np.array([counts[e] for e in eorder], dtype=np.uint32),
        "event_first": np.array([first[e] for e in eorder], dtype=np.int32),
        "event_last": np.array([last[e] for e in eorder], dtype=np.int32),
    }
    flags = np.zeros(NE, dtype=np.uint8)
    for e in range(NE):
        for t in ev_out[e]:
            m = mode_of(t)
            if m == MODE_JIT:
                flags[new_ev[e]] |= FLAG_HAS_JIT
            elif m == MODE_EMPTY:
                flags[new_ev[e]] |= FLAG_HAS_EMPTY
    out["event_flags"] = flags
    worker = np.full(NT, -1, dtype=np.int16)
    lists = [[] for _ in range(W)]
    k = 0
    for i in range(NT):
        if out["task_mode"][i] == MODE_AOT:
            worker[i] = k % W
            lists[k % W].append(i)
            k += 1
    out["task_worker"] = worker
    out["aot_offsets"] = np.array(np.cumsum([0] + [len(x) for x in lists]), dtype=np.uint32)
    out["aot_tasks"] = np.array([i for x in lists for i in x], dtype=np.uint32)
    out["header"] = dict(NT=NT, NE=NE, root=new_ev[root], end=new_ev[end], n_fused=len(fused),
                         n_empty=n_empty, n_rewrites=len(ev_in) - 2 - len(fused))
    return out


def build(cfg, B, P, prm: Params):
    """The whole spec for a decoder: decompose, then canonicalise."""
    tasks = decompose(cfg, B, P, prm)
    return canonicalize(tasks, prm.W, prm.jit_attn, prm.jit_all, prm.fusion), tasks


# ----------------------------------------------------------------------------- checker
def check_semantics(g, tasks=None, closure=True):
    """Checks that hold for any correct tGraph, independent of the spec's
    numbering choices.  Raises AssertionError on the first violation.

    * each task has exactly one dependent and one triggering event, neither
      is the wrong end of the graph;
    * each event's dependent tasks are exactly ``[first, last]`` (contiguity);
    * ``counts(e)`` equals the number of tasks that trigger ``e``;
    * the linear order is topological; AOT lists increase; modes/flags agree;
    * with ``tasks`` given and ``closure``: over real tasks, "c waits for p"
      in the final graph equals the transitive closure of the overlap edges.
    """
    NT = len(g["task_type"]); NE = len(g["event_counts"])
    hdr = g["header"]
    root, end = hdr["root"], hdr["end"]
    dep = g["task_dep"].astype(np.int64); trig = g["task_trig"].astype(np.int64)
    assert np.all((dep >= 0) & (dep < NE)) and np.all((trig >= 0) & (trig < NE)), "event index out of range"
    assert not np.any(dep == end) and not np.any(trig == root), "a task waits on the end or triggers the root"
    # contiguity
    first = g["event_first"].astype(np.int64); last = g["event_last"].astype(np.int64)
    for e in range(NE):
        idx = np.nonzero(dep == e)[0]
        if len(idx) == 0:
            assert first[e] == last[e] + 1, f"contiguity: event {e} has no consumers but range [{first[e]}, {last[e]}]"
        else:
            assert idx[0] == first[e] and idx[-1] == last[e] and len(idx) == last[e] - first[e] + 1, \
                f"contiguity: consumers of event {e} are not [first, last]"
    # counts
    cnt = np.bincount(trig, minlength=NE)
    assert np.array_equal(cnt, g["event_counts"].astype(np.int64)), "counts: an event's count differs from its producers"
    assert g["event_counts"][root] == 0, "counts: the root event has producers"
    # topological: every producer of dep(t) precedes t
    maxprod = np.full(NE, -1, dtype=np.int64)
    np.maximum.at(maxprod, trig, np.arange(NT))
    assert np.all(maxprod[dep] < np.arange(NT)), "topological: a task precedes a producer of its event"
    # degree-1 structure and modes
    tt = g["task_type"]; md = g["task_mode"]
    # EMPTY exactly the empties; the root's consumers AOT; either JIT tasks
    # are attention tasks, all of one mode (JIT or AOT), or every other
    # non-empty task is JIT
    assert np.all((md == MODE_EMPTY) == (tt == EMPTY)) and np.all(md[dep == root] != MODE_JIT), "modes: empty/JIT modes"
    dd = np.isin(tt, DATA_DEPENDENT)
    if np.any((md == MODE_JIT) & ~dd):
        assert np.all(md[(tt != EMPTY) & (dep != root)] == MODE_JIT), "modes: mixed JIT policy"
    else:
        assert len(set(md[dd & (dep != root)].tolist())) <= 1, "modes: mixed attention modes"
    for e in range(NE):
        cons = md[first[e]:last[e] + 1]
        f = (FLAG_HAS_JIT if np.any(cons == MODE_JIT) else 0) | (FLAG_HAS_EMPTY if np.any(cons == MODE_EMPTY) else 0)
        assert g["event_flags"][e] == f, f"flags: event {e}"
    # AOT lists
    off = g["aot_offsets"].astype(np.int64); lst = g["aot_tasks"].astype(np.int64)
    W = len(off) - 1
    assert off[0] == 0 and off[-1] == len(lst) == int(np.sum(md == MODE_AOT)), "aot: list sizes"
    for w in range(W):
        seg = lst[off[w]:off[w + 1]]
        assert np.all(np.diff(seg) > 0), f"aot: list of worker {w} not increasing"
        assert np.all(g["task_worker"][seg] == w), f"aot: task_worker disagrees with list {w}"
    assert np.all((g["task_worker"] >= 0) == (md == MODE_AOT)), "aot: task_worker on a non-AOT task"
    if tasks is not None and closure:
        _check_closure(g, tasks)


def _check_closure(g, tasks):
    N = len(tasks)
    P = producer_sets(tasks)
    # closure of the original overlap edges (program order is topological)
    reach = [0] * N
    for c in range(N):
        r = 0
        for p in P[c]:
            r |= reach[p] | (1 << p)
        reach[c] = r
    # closure of the final graph, restricted to real tasks, in original ids
    NT = len(g["task_type"])
    orig = g["task_orig"]; dep = g["task_dep"]; trig = g["task_trig"]
    prods = {}
    for t in range(NT):
        prods.setdefault(int(trig[t]), []).append(t)
    waits = [0] * NT
    for t in range(NT):
        r = 0
        for p in prods.get(int(dep[t]), []):
            r |= waits[p]
            if orig[p] >= 0:
                r |= 1 << int(orig[p])
        waits[t] = r
    seen = 0
    for t in range(NT):
        if orig[t] >= 0:
            assert waits[t] == reach[int(orig[t])], f"closure differs at task {t} (orig {orig[t]})"
            seen += 1
    assert seen == N, "closure: a real task is missing"


def generic_tasks(specs, regions):
    """Tasks for the generic canonicalisation entry: ``specs`` is a list of
    ``(type, layer, c0, c1, c2)``; ``regions`` a list of
    ``(task, is_out, tensor, lo[4], hi[4])``."""
    tasks = [dict(type=s[0], layer=s[1], coords=tuple(s[2:5]), ins=[], outs=[]) for s in specs]
    for (t, is_out, tn, lo, hi) in regions:
        tasks[t]["outs" if is_out else "ins"].append((tn, tuple(lo), tuple(hi)))
    return tasks
