"""Pins for the tGraph oracle (CPU only).

* the hand-derived tiny-decoder example (counts, sizes, start of the linear order);
* rewrite-count identities;
* semantic checks that do not depend on the spec's numbering (degree <= 1,
  contiguity, counts, topological order, closure equality) on the decoder
  graphs and on randomly generated programs with misaligned tilings.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import synth
from oracle import tgraph as tg

TINY_PRM = tg.Params(W=8, q=64, T_qkv=8, T_o=4, T_gu=11, T_down=4, T_lm=16, S_attn=4)


def tiny():
    return tg.build(synth.SHAPES["tiny"].cfg(), 1, 16, TINY_PRM)


def test_tiny_worked_example_sizes():
    g, tasks = tiny()
    h = g["header"]
    # Hand count (batch 1, so the norms run inside the projection tiles): per layer
    # 8 QKV + 2 groups x 4 splits ATTN + 4 OPROJ + 11 GATEUP + 4 DOWN = 35 tasks; 2 layers,
    # 16 LM-head tiles and ARGMAX give 87.  Fused events: layer 0 {2 ATTN groups, OPROJ,
    # GATEUP, DOWN}, layer 1 the same plus its QKV event, then LM head and ARGMAX = 13.
    # QKV tile 0 (also stores the residual for GATEUP) and GATEUP tile 0 (also stores the
    # residual for the next layer / LM head) each feed two events: 4 rewrites, 8 empties.
    assert len(tasks) == 87
    assert sum(1 for t in tasks if t["layer"] == 0) == 35
    assert h["n_fused"] == 13 and h["n_rewrites"] == 4 and h["n_empty"] == 8
    assert h["NT"] == 95 and h["NE"] == 19 and h["root"] == 0 and h["end"] == 18


def test_tiny_worked_example_order_and_counts():
    g, _ = tiny()
    T = tg
    tt = list(g["task_type"])
    # layer-0 QKV tiles are the sources; the empties of QKV tile 0 follow them
    expect = [T.QKV] * 8 + [T.EMPTY] * 2 + [T.ATTN] * 8 + [T.OPROJ] * 4 + [T.GATEUP] * 11 + [T.EMPTY] * 2 + \
        [T.DOWN] * 4 + [T.QKV] * 8
    assert tt[:len(expect)] == expect
    cnt = g["event_counts"]; dep = g["task_dep"]
    c = lambda i: int(cnt[dep[i]])
    assert all(c(i) == 0 for i in range(8))      # root
    assert c(8) == 1 and c(9) == 1               # e' of QKV tile 0
    assert all(c(i) == 4 for i in range(10, 18))  # a split waits for the 4 projection tiles of its group
    assert c(18) == 8                            # O projection waits for all 8 splits (any may combine)
    assert c(22) == 5                            # GATEUP: 4 O tiles + the empty standing in for QKV tile 0
    assert c(35) == 11                           # DOWN waits for the 11 gate/up tiles
    assert c(39) == 5                            # next QKV: 4 DOWN tiles + the empty for GATEUP tile 0
    # the two empties of QKV tile 0 feed, in order, the group-0 attention event and the GATEUP event
    assert g["task_orig"][8] == -1 and g["task_orig"][9] == -2
    # (group 1's event completes with tile 7, before group 0's completes through empty 8, so the
    # BFS places group 1's splits at 10..13 and group 0's at 14..17)
    assert g["event_first"][g["task_trig"][8]] == 14
    assert [tuple(g["task_coords"][i]) for i in (10, 14)] == [(0, 1, 0), (0, 0, 0)]
    assert g["task_type"][g["event_first"][g["task_trig"][9]]] == T.GATEUP
    # ATTN tasks are JIT, empties EMPTY, all else AOT; the AOT worker is round-robin in linear order
    aot = [i for i in range(len(tt)) if g["task_mode"][i] == T.MODE_AOT]
    assert [int(g["task_worker"][i]) for i in aot] == [k % 8 for k in range(len(aot))]
    lm = tt.index(T.LMHEAD)
    assert c(lm) == 5                            # last DOWN tiles + the empty of the last GATEUP tile 0
    argmax = tt.index(T.ARGMAX)
    assert c(argmax) == 16 and g["event_counts"][g["header"]["end"]] == 1
    tg.check_semantics(g, _, closure=True)


def test_tiny_worked_example_batch3_keeps_norm_tasks():
    g, tasks = tg.build(synth.SHAPES["tiny"].cfg(), 3, 16, TINY_PRM)
    tt = list(g["task_type"])
    T_EMPTY = tg.EMPTY
    # Hand count: 3 EMBED (one per request) + per layer (3 ATTN_NORM, 8 QKV, 2 kv groups x 4 attention
    # slots, 4 OPROJ, 3 MLP_NORM, 11 GATEUP, 4 DOWN) = 3 + 2 x 41, + 3 FINAL_NORM + 16 LM + ARGMAX = 105.
    assert len(tasks) == 105
    assert [tuple(t["coords"]) for t in tasks if t["type"] == tg.ATTN_NORM][:3] == [(0, 0, 0), (1, 0, 0), (2, 0, 0)]
    # Each norm task feeds two events: the next projection's (all B norm tasks) and the next norm's
    # (all B norm tasks + the projection tiles after them): 2 x (3 + 3) rewrites, 2 empties each.
    # Fused events per layer: [ATTN_NORM], QKV, 2 attention groups, OPROJ, MLP_NORM, GATEUP, DOWN = 8;
    # then FINAL_NORM, LM head, ARGMAX: 19.
    h = g["header"]
    assert h["n_rewrites"] == 12 and h["n_empty"] == 24 and tt.count(T_EMPTY) == 24 and h["n_fused"] == 19
    assert h["NT"] == 105 + 24 and h["NE"] == 19 + 12 + 2
    assert tt[:12] == [tg.EMBED] * 3 + [tg.ATTN_NORM] * 3 + [T_EMPTY] * 6
    cnt = g["event_counts"]; dep = g["task_dep"]
    assert all(int(cnt[dep[i]]) == 3 for i in range(3, 6))   # every layer-0 norm waits for the 3 embeddings
    assert int(cnt[dep[12]]) == 3 and tt[12] == tg.QKV         # QKV waits for the 3 norms (via their empties)
    assert tg.QKNORM_ROPE not in tt and tg.COMBINE not in tt
    tg.check_semantics(g, tasks, closure=True)


def test_tiny_worked_example_aot_attention():
    # the same graph with attention placed ahead of time: identical tasks and events, no JIT flag,
    # and the round-robin placement now runs over the attention tasks too
    from dataclasses import replace
    g, _ = tiny()
    ga, tasks = tg.build(synth.SHAPES["tiny"].cfg(), 1, 16, replace(TINY_PRM, jit_attn=False))
    for k in ("task_type", "task_dep", "task_trig", "event_counts", "event_first", "event_last"):
        assert np.array_equal(g[k], ga[k]), k
    assert not np.any(ga["task_mode"] == tg.MODE_JIT) and not np.any(ga["event_flags"] & tg.FLAG_HAS_JIT)
    aot = [i for i in range(len(ga["task_type"])) if ga["task_mode"][i] == tg.MODE_AOT]
    assert len(aot) == 87 and [int(ga["task_worker"][i]) for i in aot] == [k % 8 for k in range(87)]
    tg.check_semantics(ga, tasks, closure=True)


def test_rewrite_identities():
    g, tasks = tiny()
    P = tg.producer_sets(tasks)
    groups = {}
    for c_, p in enumerate(P):
        if p:
            groups.setdefault(frozenset(p), set()).add(c_)
    fanout = [sum(1 for k in groups if t in k) for t in range(len(tasks))]
    assert g["header"]["n_empty"] == sum(f for f in fanout if f >= 2)
    assert g["header"]["NE"] == len(groups) + sum(1 for f in fanout if f >= 2) + 2


@pytest.mark.parametrize("name,B,S", [("tiny", 3, 4), ("qwen3_0p6b", 1, 16), ("qwen3_8b", 2, 8)])
def test_decoder_graph_semantics_small_cuts(name, B, S):
    s = synth.SHAPES[name].with_(n_layers=2, vocab=4096)
    cfg = s.cfg()
    W = 24
    hkv = s.n_kv_heads
    prm = tg.Params(W=W, q=1 if B == 1 else 16, T_qkv=(W // hkv) * hkv, T_o=W, T_gu=W, T_down=W, T_lm=W, S_attn=S)
    g, tasks = tg.build(cfg, B, s.page_size, prm)
    tg.check_semantics(g, tasks, closure=True)


@pytest.mark.parametrize("name", ["qwen3_0p6b", "qwen3_8b", "qwen3_8b_b16", "qwen3_32b"])
def test_full_graph_invariants(name):
    s = synth.SHAPES[name]
    W = 252
    prm = tg.Params(W=W, q=1 if s.batch == 1 else 16, T_qkv=(W // s.n_kv_heads) * s.n_kv_heads, T_o=W, T_gu=W,
                    T_down=W, T_lm=W, S_attn=16 if s.batch == 1 else 31)
    g, _ = tg.build(s.cfg(), s.batch, s.page_size, prm)
    tg.check_semantics(g, None)
    h = g["header"]
    # two tasks per layer (the residual keepers) fan out to two events at batch 1, the 2 B norm
    # tasks per layer at batch B > 1; each such task gets two empties
    per_layer = 2 if s.batch == 1 else 2 * s.batch
    assert h["n_empty"] == 2 * per_layer * s.n_layers
    assert h["n_empty"] / h["NT"] < (0.01 if s.batch == 1 else 0.05)   # "deep, not wide"


# ------------------------------------------------------------------ random programs
@st.composite
def programs(draw):
    n_ops = draw(st.integers(1, 5))
    tensors = []          # (n_dims, shape)
    tasks = []            # (type, layer, c0, c1, c2)
    regions = []          # (task, is_out, tensor, lo, hi)
    produced = []
    for op in range(n_ops):
        nd = draw(st.integers(1, 2))
        shape = tuple(draw(st.integers(1, 9)) for _ in range(nd))
        out_t = len(tensors)
        tensors.append(shape)
        # tile the output along dim 0 with random cut points
        cuts = sorted(set(draw(st.lists(st.integers(1, shape[0] - 1), max_size=3)) if shape[0] > 1 else []))
        bounds = [0] + cuts + [shape[0]]
        tp = draw(st.sampled_from([tg.QKV, tg.ATTN, tg.OPROJ, tg.MLP_NORM, tg.COMBINE]))
        srcs = draw(st.lists(st.sampled_from(produced), max_size=2, unique=True)) if produced else []
        for j in range(len(bounds) - 1):
            tid = len(tasks)
            tasks.append((tp, op, j, 0, 0))
            lo = [bounds[j]] + [0] * (nd - 1); hi = [bounds[j + 1]] + list(shape[1:])
            regions.append((tid, 1, out_t, tuple(lo) + (0,) * (4 - nd), tuple(hi) + (1,) * (4 - nd)))
            for s_ in srcs:
                sh = tensors[s_]
                lo = [draw(st.integers(0, x - 1)) for x in sh]
                hi = [draw(st.integers(l_ + 1, x)) for l_, x in zip(lo, sh)]
                k = len(sh)
                regions.append((tid, 0, s_, tuple(lo) + (0,) * (4 - k), tuple(hi) + (1,) * (4 - k)))
        produced.append(out_t)
    W = draw(st.integers(1, 4))
    return tasks, regions, W


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(programs())
def test_random_programs_preserve_every_wait(prog):
    specs, regions, W = prog
    tasks = tg.generic_tasks(specs, regions)
    g = tg.canonicalize(tasks, W)
    tg.check_semantics(g, tasks, closure=True)
    assert g["header"]["NT"] == len(tasks) + g["header"]["n_empty"]


# ------------------------------------------------------------------ the checker must reject wrong graphs
# Each case breaks one property that MPK summary section 4 ("6 minimum checks") requires of a
# canonical tGraph and asserts that check_semantics rejects it, naming the property.
def _raises(g, tasks, what):
    with pytest.raises(AssertionError, match=what):
        tg.check_semantics(g, tasks, closure=tasks is not None)


def _copy(g):
    return {k: (v.copy() if isinstance(v, np.ndarray) else dict(v) if isinstance(v, dict) else v) for k, v in g.items()}


def test_checker_rejects_a_dropped_wait():
    # O-projection tile 0 of layer 0 declares only kv group 0's part of the attention output, so the
    # graph built from it lets the tile start before group 1's splits: a wait the true boxes need
    g, tasks = tiny()
    bad = [dict(t, ins=list(t["ins"])) for t in tasks]
    k = next(i for i, t in enumerate(bad) if t["type"] == tg.OPROJ and t["layer"] == 0)
    tn, lo, hi = bad[k]["ins"][0]
    G_d = 2 * 64                      # tiny: 2 query heads of 64 per kv group
    bad[k]["ins"][0] = (tn, lo, (hi[0], G_d) + tuple(hi[2:]))
    gb = tg.canonicalize(bad, TINY_PRM.W, TINY_PRM.jit_attn)
    tg.check_semantics(gb, bad, closure=True)     # consistent with its own (wrong) boxes
    _raises(gb, tasks, "closure")


def test_checker_rejects_an_added_wait():
    # the operator-level graph makes every attention split wait for all q/k/v tiles; against the
    # fine boxes that is a wait no overlap implies
    from dataclasses import replace
    _, fine = tiny()
    gc, coarse = tg.build(synth.SHAPES["tiny"].cfg(), 1, 16, replace(TINY_PRM, coarse=True))
    tg.check_semantics(gc, coarse, closure=True)
    _raises(gc, fine, "closure")


def test_checker_rejects_a_broken_range():
    g, tasks = tiny()
    e = int(np.argmax(g["event_last"] - g["event_first"]))     # an event with several consumers
    bad = _copy(g)
    bad["event_last"][e] -= 1
    _raises(bad, None, "contiguity")
    bad = _copy(g)
    bad["event_first"][e] += 1
    _raises(bad, None, "contiguity")


def test_checker_rejects_a_wrong_count():
    g, tasks = tiny()
    for e in (int(g["task_dep"][20]), int(g["header"]["end"])):
        bad = _copy(g)
        bad["event_counts"][e] += 1
        _raises(bad, None, "counts")


def test_checker_rejects_wrong_flags_and_aot_lists():
    g, _ = tiny()
    bad = _copy(g)
    bad["event_flags"][int(g["task_dep"][8])] ^= tg.FLAG_HAS_EMPTY
    _raises(bad, None, "flags")
    bad = _copy(g)
    lst = bad["aot_tasks"]
    lst[0], lst[1] = lst[1], lst[0]
    _raises(bad, None, "aot")


def test_checker_rejects_a_non_topological_order():
    # two tasks: linear task 0 waits on event 1, which linear task 1 triggers; task 1 waits on
    # the root (event 0), task 0 triggers the end (event 2).  Ranges and counts are consistent;
    # only the order is wrong.
    g = {"task_type": np.array([tg.QKV, tg.QKV], np.uint8), "task_mode": np.zeros(2, np.uint8),
         "task_dep": np.array([1, 0], np.int32), "task_trig": np.array([2, 1], np.int32),
         "task_worker": np.array([0, 0], np.int16), "event_counts": np.array([0, 1, 1], np.uint32),
         "event_first": np.array([1, 0, 3], np.int32), "event_last": np.array([1, 0, 2], np.int32),
         "event_flags": np.zeros(3, np.uint8), "aot_offsets": np.array([0, 2], np.uint32),
         "aot_tasks": np.array([0, 1], np.uint32), "header": dict(root=0, end=2)}
    _raises(g, None, "topological")
    ok = _copy(g)   # the same two tasks in the right order pass
    ok.update(task_dep=np.array([0, 1], np.int32), task_trig=np.array([1, 2], np.int32),
              event_first=np.array([0, 1, 2], np.int32), event_last=np.array([0, 1, 1], np.int32))
    tg.check_semantics(ok)


# ------------------------------------------------------------------ top-2 gap
def test_top2_gap_hand_values():
    from oracle import numerics as on
    rows = np.array([[1.0, 3.0, 2.0],        # 3 - 2
                     [5.0, 5.0, 1.0],        # a tie at the top: 0
                     [-3.0, -1.0, -2.0],     # negatives: -1 - (-2)
                     [0.5, 0.5, 0.5],        # all equal: 0
                     [7.0, -4.0, 2.5]])      # 7 - 2.5
    np.testing.assert_array_equal(on.top2_gap(rows), [1.0, 0.0, 1.0, 0.0, 4.5])
    assert on.top2_gap(np.array([2.0, 10.0])) == 8.0


# ------------------------------------------------------------------ no fusion: the fan-in rewrite
def _two_by_two():
    """Operator A (tiles A0, A1) writes tensor 0; operator B (tiles B0, B1) reads all of it."""
    specs = [(tg.QKV, 0, 0, 0, 0), (tg.QKV, 0, 1, 0, 0), (tg.OPROJ, 0, 0, 0, 0), (tg.OPROJ, 0, 1, 0, 0)]
    regions = [(0, 1, 0, (0, 0, 0, 0), (1, 4, 1, 1)), (1, 1, 0, (0, 4, 0, 0), (1, 8, 1, 1)),
               (2, 0, 0, (0, 0, 0, 0), (1, 8, 1, 1)), (3, 0, 0, (0, 0, 0, 0), (1, 8, 1, 1)),
               (2, 1, 1, (0, 0, 0, 0), (1, 1, 1, 1)), (3, 1, 1, (0, 1, 0, 0), (1, 2, 1, 1))]
    return specs, regions


def test_fusion_off_hand_example():
    # Hand derivation.  Fused (Def 4.1 then 4.2): one event {A0, A1} -> {B0, B1}; with root and end
    # NE = 3, NT = 4.  Without fusion: 4 edge events pre-ordered (B0,A0) (B0,A1) (B1,A0) (B1,A1);
    # A0 and A1 each fan out to 2 (e' + 2 empties), B0 and B1 each fan in from 2 (e' + 2 empties):
    # 8 empties, NE = 4 + 4 + 2 = 10.  Empties are numbered A0's two, A1's two (fan-out, coords (i,0)),
    # then B0's two, B1's two (fan-in, coords (i,1)).  BFS: root -> A0, A1; e'(A0) -> its empties,
    # which fire (B0,A0), (B1,A0); e'(A1) -> its empties, firing (B0,A1), (B1,A1); those four events
    # place the fan-in empties of B0, B1, B0, B1; then e'(B0) -> B0, e'(B1) -> B1.
    specs, regions = _two_by_two()
    tasks = tg.generic_tasks(specs, regions)
    gf = tg.canonicalize(tasks, 2)
    assert (gf["header"]["NT"], gf["header"]["NE"], gf["header"]["n_empty"]) == (4, 3, 0)
    g = tg.canonicalize(tasks, 2, fusion=tg.FUSION_OFF)
    h = g["header"]
    assert (h["NT"], h["NE"], h["n_fused"], h["n_rewrites"], h["n_empty"]) == (12, 10, 4, 4, 8)
    assert g["task_orig"].tolist() == [0, 1, -1, -2, -3, -4, -5, -7, -6, -8, 2, 3]
    assert [tuple(c[:2]) for c in g["task_coords"][2:10]] == [(0, 0), (1, 0), (0, 0), (1, 0),
                                                              (0, 1), (0, 1), (1, 1), (1, 1)]
    cnt = g["event_counts"][g["task_dep"]]
    assert cnt.tolist() == [0, 0, 1, 1, 1, 1, 1, 1, 1, 1, 2, 2]   # the fan-in e' of B0 and B1 count 2
    assert g["event_counts"][h["end"]] == 2
    tg.check_semantics(g, tasks, closure=True)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(programs())
def test_random_programs_without_fusion_preserve_every_wait(prog):
    specs, regions, W = prog
    tasks = tg.generic_tasks(specs, regions)
    g = tg.canonicalize(tasks, W, fusion=tg.FUSION_OFF)
    tg.check_semantics(g, tasks, closure=True)
    P = tg.producer_sets(tasks)
    fan_in = sum(len(p) for p in P if len(p) >= 2)
    fan_out = sum(n for n in np.bincount([x for p in P for x in p], minlength=len(tasks)) if n >= 2)
    assert g["header"]["n_empty"] == fan_in + fan_out
    assert g["header"]["n_fused"] == sum(len(p) for p in P)


def test_tiny_decoder_without_fusion():
    from dataclasses import replace
    g, tasks = tg.build(synth.SHAPES["tiny"].cfg(), 1, 16, replace(TINY_PRM, fusion=tg.FUSION_OFF))
    tg.check_semantics(g, tasks, closure=True)
    gf, _ = tiny()
    assert g["header"]["n_empty"] > 10 * gf["header"]["n_empty"]   # no fusion: a wide graph
