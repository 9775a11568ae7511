"""GPU parity: the decode step through the C ABI against the oracle.

Every case runs the persistent mega-kernel (and the kernel-per-operator
baseline where noted) on seeded synthetic inputs and compares with the CPU
oracle: logits within |d| <= 2e-2 + 2e-2 |ref|, greedy ids equal wherever the
oracle's top-2 gap exceeds 1e-2, and the KV-cache slot the step writes equal
to the oracle's new k/v rounded to bf16.
"""
import numpy as np
import pytest
import torch

import synth
import task_graph_runtime_amd as mpk
from oracle import numerics as on
from tests._util import run_oracle, bf16_round

pytestmark = pytest.mark.gpu

ATOL, RTOL, GAP = 2e-2, 2e-2, 1e-2


def say(*a):
    print("[case]", *a, flush=True)


def device_inputs(shape, seed=0, gamma="ones", seq_lens=None):
    inp = synth.make_inputs(shape, seed=seed, device="cuda", gamma=gamma, seq_lens=seq_lens)
    inp["kv"]["page_table_dev"] = inp["kv"]["page_table"].cuda()
    inp["token_ids_dev"] = inp["token_ids"].cuda()
    inp["seq_lens_dev"] = inp["seq_lens"].cuda()
    return inp


class Runner:
    def __init__(self, inp, params=None):
        s = inp["shape"]
        self.inp = inp
        self.g = mpk.TGraph(s.cfg(), s.batch, s.page_size, params or {})
        self.w = mpk.Weights(inp["weights"])
        kv = inp["kv"]
        self.kv = mpk.KV(kv["k_pool"], kv["v_pool"], kv["page_table_dev"])
        self.logits = torch.full((s.batch, s.vocab), float("nan"), device="cuda", dtype=torch.float32)
        self.next = torch.full((s.batch,), -1, device="cuda", dtype=torch.int32)

    def run(self, mode="mega"):
        self.logits.fill_(float("nan"))
        self.next.fill_(-1)
        args = (self.w, self.inp["token_ids_dev"], self.kv, self.inp["seq_lens_dev"], self.logits, self.next)
        if mode == "mega":
            self.g.decode_step(*args)
        else:
            self.g.decode_step_baseline(*args, use_hipgraph=(mode == "graph"))
        torch.cuda.synchronize()
        st = self.g.status()
        assert st["code"] == 0, st
        return self.logits.cpu().numpy(), self.next.cpu().numpy()


def check(logits, nxt, ref, ref_next):
    assert np.all(np.isfinite(logits))
    err = np.abs(logits - ref)
    tol = ATOL + RTOL * np.abs(ref)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} logits out of tolerance; max |d| = {err.max():.3g}"
    gap = on.top2_gap(ref)
    m = gap > GAP
    assert np.array_equal(nxt[m], ref_next[m]), (nxt, ref_next, gap)
    return float(err.max())


def check_cache(inp, cap):
    s = inp["shape"]
    kv = inp["kv"]
    P = s.page_size
    for l in range(s.n_layers):
        for b in range(s.batch):
            Lb = int(inp["seq_lens"][b])
            pid = int(kv["page_table"][b, Lb // P])
            for pool, name in ((kv["k_pool"], "k_new"), (kv["v_pool"], "v_new")):
                got = pool[l, pid, :, Lb % P, :].float().cpu().numpy()
                want = bf16_round(cap[l][name][b])
                # same bound as the logits: both sides round to bf16 from slightly different fp32 values
                np.testing.assert_allclose(got, want, rtol=RTOL, atol=ATOL, err_msg=f"{name} l={l} b={b}")


TINY = synth.SHAPES["tiny"]


@pytest.mark.parametrize("mode", ["mega", "base", "graph"])
def test_tiny_batch1(mode):
    say("tiny B=1", mode)
    inp = device_inputs(TINY, seed=0, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    r = Runner(inp)
    logits, nxt = r.run(mode)
    check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.parametrize("B", [1, 2])
def test_tiny_intermediates_layer_by_layer(B):
    """Every library-owned intermediate against the oracle's, layer by layer.
    B = 1 runs the fused-norm graph (residuals stored by the first QKV / GATEUP
    tile); B = 2 the graph with norm tasks (e, h, h2 and hf exist too)."""
    say("tiny intermediates", B)
    s = TINY.with_(batch=B, ctx_range=(3, 40), ctx=0)
    inp = device_inputs(s, seed=4, gamma="uniform")
    cap = {}
    run_oracle(inp, capture=cap)
    r = Runner(inp)
    r.run("mega")
    g = r.g
    H, F = s.hidden, s.ffn
    hq, hkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim
    G = hq // hkv
    # q/k/v, output and down projections: the sum of their k-split planes
    p = g.header()["params"]
    Kq, Ko, Kd = p["k_qkv"], p["k_o"], p["k_down"]
    if B > 1:
        assert (Kq, Ko, Kd) != (1, 1, 1)
        np.testing.assert_allclose(g.read_tensor(0, (B, H), np.float32), cap["embed"], rtol=0, atol=0)
    for l in range(s.n_layers):
        t = lambda k: 5 + mpk._binding.LAYER_TENSORS * l + k
        c = cap[l]
        np.testing.assert_allclose(g.read_tensor(t(0), (B, H), np.float32), c["r"], rtol=2e-2, atol=2e-2)
        if B > 1:
            np.testing.assert_allclose(g.read_tensor(t(1), (B, H), np.float32), c["h"], rtol=2e-2, atol=2e-2)
            np.testing.assert_allclose(g.read_tensor(t(10), (B, H), np.float32), c["h2"], rtol=3e-2, atol=3e-2)
        qkv = g.read_tensor(t(2), (Kq, B, hkv, (G + 2) * d), np.float32).sum(axis=0)
        # oracle qkv is [q heads | k heads | v heads]; the library's is group-major
        oq = c["qkv"][:, :hq * d].reshape(B, hkv, G * d)
        ok = c["qkv"][:, hq * d:(hq + hkv) * d].reshape(B, hkv, d)
        ov = c["qkv"][:, (hq + hkv) * d:].reshape(B, hkv, d)
        np.testing.assert_allclose(qkv, np.concatenate([oq, ok, ov], axis=2), rtol=3e-2, atol=3e-2)
        np.testing.assert_allclose(g.read_tensor(t(7), (B, hq * d), np.float32), c["attn"], rtol=3e-2, atol=3e-2)
        np.testing.assert_allclose(g.read_tensor(t(8), (Ko, B, H), np.float32).sum(axis=0), c["o"], rtol=3e-2,
                                   atol=3e-2)
        np.testing.assert_allclose(g.read_tensor(t(9), (B, H), np.float32), c["s"], rtol=3e-2, atol=3e-2)
        np.testing.assert_allclose(g.read_tensor(t(11), (B, F), np.float32), c["a"], rtol=3e-2, atol=3e-2)
        np.testing.assert_allclose(g.read_tensor(t(12), (Kd, B, H), np.float32).sum(axis=0), c["d"], rtol=3e-2,
                                   atol=3e-2)
    if B > 1:
        np.testing.assert_allclose(g.read_tensor(1, (B, H), np.float32), cap["hf"], rtol=3e-2, atol=3e-2)
    check_cache(inp, cap)


@pytest.mark.parametrize("K", [(1, 1, 1), (3, 2, 4), (2, 5, 3)])
@pytest.mark.parametrize("mode", ["mega", "base"])
def test_tiny_k_split(K, mode):
    """Batch 3 with the q/k/v, output and down projections split along their
    contraction into K ranges (the readers add the planes)."""
    s = TINY.with_(batch=3, ctx_range=(3, 120), ctx=0)
    say("tiny k-split", K, mode)
    inp = device_inputs(s, seed=31, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    r = Runner(inp, dict(k_qkv=K[0], k_o=K[1], k_down=K[2]))
    logits, nxt = r.run(mode)
    check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("params", [dict(attn_jit=3), dict(attn_jit=1), dict(weight_preload=2), dict(coarse_events=1),
                                    dict(weight_preload=3), dict(weight_preload=3, attn_jit=1)])
def test_tiny_scheduling_ablations(B, params):
    """The ablation builds: every task JIT, attention JIT, no weight pre-load,
    the operator-level graph and the paged lookahead (its own kernel; with
    attention JIT only the projections are staged), each against the oracle."""
    s = TINY.with_(batch=B, ctx_range=(3, 120), ctx=0)
    say("tiny ablation", B, params)
    inp = device_inputs(s, seed=51 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    logits, nxt = Runner(inp, params).run("mega")
    check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.parametrize("B", [1, 3])
def test_tiny_eight_query_heads_per_group(B):
    """The G = 8 attention body (32 lanes per key row, as at the 32B shape) on a
    small decoder: 16 q heads over 2 kv heads of 128 dims."""
    s = TINY.with_(n_q_heads=16, n_kv_heads=2, head_dim=128, qk_norm=True, batch=B, ctx_range=(30, 250), ctx=0)
    say("tiny G=8", B)
    inp = device_inputs(s, seed=21 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    logits, nxt = Runner(inp).run("mega")
    check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.parametrize("B,lens", [
    (3, [0, 15, 16]),              # empty context; new token ends a page; new token opens a page
    (4, [1, 31, 100, 255]),        # 255 = max_seq_len - 1: the last slot
    (16, None),                    # batch 16, ragged lengths
    (1, [0]),                      # the first token of a request: attention over itself alone
    (16, [0] * 16),                # a full batch of first tokens
    (16, [255] * 16),              # a full batch at the last slot
])
@pytest.mark.parametrize("mode", ["mega", "base"])
def test_tiny_ragged(B, lens, mode):
    s = TINY.with_(batch=B, ctx_range=(0, 255), ctx=0)
    say("tiny ragged", B, lens, mode)
    inp = device_inputs(s, seed=7 + B, gamma="uniform", seq_lens=lens)
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    logits, nxt = Runner(inp).run(mode)
    check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.parametrize("params", [
    dict(n_workers=8, quantum=64, t_qkv=8, t_o=4, t_gu=11, t_down=4, t_lm=16, s_attn=4),   # the worked example
    dict(n_workers=3, n_sched_waves=4, s_attn=2),                                             # few workers, one split each
    dict(n_workers=200, s_attn=9, t_lm=1000, quantum=1),                                      # many tiles, odd split
])
def test_tiny_build_params(params):
    say("tiny params", params)
    s = TINY.with_(batch=2, ctx_range=(10, 200), ctx=0)
    inp = device_inputs(s, seed=21)
    ref, ref_next = run_oracle(inp)
    logits, nxt = Runner(inp, params).run("mega")
    check(logits, nxt, ref, ref_next)


def test_tiny_repeated_steps_are_stable():
    say("tiny repeated steps")
    inp = device_inputs(TINY, seed=2)
    ref, ref_next = run_oracle(inp)
    r = Runner(inp)
    outs = []
    for mode in ["mega", "mega", "base", "mega", "graph", "graph", "mega"]:
        logits, nxt = r.run(mode)
        check(logits, nxt, ref, ref_next)
        outs.append(logits)
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("B", [1, 3, 16])
def test_tiny_alternating_inputs(B):
    """Steps of one graph alternate between two token sets: each step matches
    its own oracle, so nothing a step reads is left over from the step before
    (task-to-task data that projection tiles read through the L2)."""
    s = TINY.with_(batch=B, ctx_range=(3, 120), ctx=0)
    say("tiny alternating inputs", B)
    inp = device_inputs(s, seed=41 + B, gamma="uniform")
    ids = [inp["token_ids"].clone(), (inp["token_ids"] * 7 + 13) % s.vocab]
    refs = []
    for t in ids:
        inp["token_ids"] = t
        refs.append(run_oracle(inp))
    r = Runner(inp)
    for k in [0, 1, 0, 1, 1, 0]:
        r.inp["token_ids_dev"].copy_(ids[k].to(r.inp["token_ids_dev"].dtype).cuda())
        logits, nxt = r.run("mega")
        check(logits, nxt, *refs[k])


def test_watchdog_reports_timeout_and_poisons():
    say("watchdog")
    inp = device_inputs(TINY, seed=1)
    r = Runner(inp)
    r.run("mega")
    r.g.set_watchdog(1)          # a 1 ns limit: the first wait that is not already satisfied times out
    r.g.decode_step(r.w, inp["token_ids_dev"], r.kv, inp["seq_lens_dev"], r.logits, r.next)
    torch.cuda.synchronize()
    st = r.g.status()
    assert st["code"] == -5
    # poisoned: the next step exits at once and the status stays
    r.g.set_watchdog(0)
    r.g.decode_step(r.w, inp["token_ids_dev"], r.kv, inp["seq_lens_dev"], r.logits, r.next)
    assert r.g.status()["code"] == -5


def test_bad_token_id_reported_not_faulting():
    say("bad token id")
    inp = device_inputs(TINY, seed=1)
    inp["token_ids_dev"] = torch.tensor([TINY.vocab + 5], dtype=torch.int32, device="cuda")
    r = Runner(inp)
    r.g.decode_step(r.w, inp["token_ids_dev"], r.kv, inp["seq_lens_dev"], r.logits, r.next)
    torch.cuda.synchronize()
    assert r.g.status()["code"] == -1


@pytest.mark.parametrize("params", [{}, {"attn_jit": 1}])
@pytest.mark.parametrize("what", ["page", "length"])
def test_bad_page_or_length_reported_not_faulting(what, params):
    """A page id outside the pool, or a cached length past the graph's
    longest, at batch 1: the attention splits report MPK_ERR_INVALID_ARG
    (a bad page is read as page 0 and its keys are not used) and the step
    ends without a fault.  With every task ahead of time the splits' page ids
    and length are read while the workers wait; with attention JIT, by the
    splits themselves."""
    say("bad", what, params)
    inp = device_inputs(TINY, seed=1)
    if what == "page":
        n_pages = inp["kv"]["k_pool"].shape[1]
        inp["kv"]["page_table_dev"][0, 0] = n_pages + 3
    else:
        inp["seq_lens_dev"] = torch.tensor([TINY.max_seq_len + 7], dtype=torch.int32, device="cuda")
    r = Runner(inp, params)
    r.g.decode_step(r.w, inp["token_ids_dev"], r.kv, inp["seq_lens_dev"], r.logits, r.next)
    torch.cuda.synchronize()
    assert r.g.status()["code"] == -1


def test_reset_recovers_a_poisoned_graph():
    """mpk_reset_tgraph: a graph poisoned by a watchdog timeout, then by a bad
    token id, runs correct steps again after a reset (several in a row, on
    the restarted counters)."""
    say("reset after poison")
    for B in (1, 3):
        s = TINY.with_(batch=B, ctx_range=(5, 130), ctx=0) if B > 1 else TINY
        inp = device_inputs(s, seed=4)
        refs = run_oracle(inp)
        r = Runner(inp)
        r.run("mega")
        r.g.set_watchdog(1)
        r.g.decode_step(r.w, inp["token_ids_dev"], r.kv, inp["seq_lens_dev"], r.logits, r.next)
        torch.cuda.synchronize()
        assert r.g.status()["code"] == -5
        r.g.set_watchdog(0)
        r.g.reset()
        assert r.g.status()["code"] == 0
        for _ in range(3):
            logits, nxt = r.run("mega")
            check(logits, nxt, *refs)
        bad = inp["token_ids_dev"].clone()
        bad[0] = s.vocab + 7
        r.g.decode_step(r.w, bad, r.kv, inp["seq_lens_dev"], r.logits, r.next)
        torch.cuda.synchronize()
        assert r.g.status()["code"] == -1
        r.g.reset()
        for _ in range(2):
            logits, nxt = r.run("mega")
            check(logits, nxt, *refs)


# ------------------------------------------------------------------ real shapes
def _full(name, seed=0, modes=("mega",), lazy=False, builds=(), seq_lens=None):
    s = synth.SHAPES[name]
    say(name, "generate", "" if seq_lens is None else f"lengths {min(seq_lens)}..{max(seq_lens)}")
    inp = device_inputs(s, seed=seed, seq_lens=seq_lens)
    say(name, "oracle")
    ref, ref_next = run_oracle(inp, lazy=lazy, widen_on_device=True)
    r = Runner(inp)
    errs = {}
    for mode in modes:
        say(name, mode)
        logits, nxt = r.run(mode)
        errs[mode] = check(logits, nxt, ref, ref_next)
    del r
    for params in builds:   # other build parameters, mega-kernel
        say(name, params)
        r = Runner(inp, params)
        logits, nxt = r.run("mega")
        errs[str(params)] = check(logits, nxt, ref, ref_next)
        del r
    say(name, "max |d|", errs)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
def test_qwen3_0p6b_shape():
    _full("qwen3_0p6b", modes=("mega", "base"))


@pytest.mark.parametrize("s_attn", [1, 2, 4])
def test_lookahead_long_splits(s_attn):
    """The paged lookahead with attention splits of 64 to 256 cached tokens at
    head_dim 64: a split whose keys and values outgrow its page stages the
    first 32k tokens and streams the rest."""
    s = TINY.with_(ctx=250)
    say("lookahead long splits", s_attn)
    inp = device_inputs(s, seed=70 + s_attn, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    r = Runner(inp, dict(weight_preload=3, s_attn=s_attn, n_workers=8))
    for _ in range(2):
        logits, nxt = r.run("mega")
        check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.timeout(600)
def test_qwen3_8b_shape():
    # (with the scheduling and pre-load ablation builds that the measurements compare)
    _full("qwen3_8b", modes=("mega", "graph"), lazy=True,
          builds=(dict(attn_jit=3), dict(attn_jit=1), dict(weight_preload=2), dict(coarse_events=1),
                  dict(weight_preload=3)))


@pytest.mark.timeout(600)
def test_qwen3_8b_batch16_shape():
    # (default AOT attention, and the hybrid policy's JIT attention)
    _full("qwen3_8b_b16", modes=("mega",), lazy=True, builds=(dict(attn_jit=1),))


@pytest.mark.timeout(600)
def test_qwen3_8b_longest_context():
    """The 8B step at the longest cached length the shape takes (8191 =
    max_seq_len - 1): the request's page table full, the run-time split
    count at its cap, the new token in the last slot of the last page."""
    s = synth.SHAPES["qwen3_8b"]
    _full("qwen3_8b", lazy=True, seq_lens=[s.max_seq_len - 1])


@pytest.mark.timeout(900)
def test_qwen3_8b_batch16_skewed():
    """The skewed batch of the scheduling ablation -- one request at the
    longest length, fifteen at 256 -- under the default placement and under
    the hybrid policy (attention JIT)."""
    s = synth.SHAPES["qwen3_8b_b16"]
    _full("qwen3_8b_b16", lazy=True, seq_lens=[s.max_seq_len - 1] + [256] * (s.batch - 1), builds=(dict(attn_jit=1),))


@pytest.mark.timeout(900)
def test_qwen3_32b_shape():
    _full("qwen3_32b", modes=("mega",), lazy=True)


def test_trace_happens_before_every_wait():
    """Trace-based check of the runtime: every task starts after every task it
    waits for (through empty tasks) has finished, and every non-empty task runs
    exactly once per step."""
    say("trace happens-before")
    s = TINY.with_(batch=3, ctx_range=(20, 200), ctx=0)
    inp = device_inputs(s, seed=9)
    r = Runner(inp)
    r.g.set_trace(True)
    r.run("mega")
    r.run("mega")
    rec, tpu = r.g.read_trace()
    ex = r.g.export()
    NT = len(ex["task_type"])
    real = np.nonzero(ex["task_type"] != mpk._binding.TASK_EMPTY)[0]
    assert sorted(rec["task"].tolist()) == real.tolist()
    assert np.all(rec["t_wait"] <= rec["t_start"]) and np.all(rec["t_start"] <= rec["t_end"])
    start = np.zeros(NT, np.uint64); end = np.zeros(NT, np.uint64)
    start[rec["task"]] = rec["t_start"]; end[rec["task"]] = rec["t_end"]
    prods = {}
    for t in range(NT):
        prods.setdefault(int(ex["task_trig"][t]), []).append(t)

    def real_producers(e):
        out = []
        for p in prods.get(e, []):
            if ex["task_type"][p] == mpk._binding.TASK_EMPTY:
                out += real_producers(int(ex["task_dep"][p]))
            else:
                out.append(p)
        return out
    for c in real:
        for p in real_producers(int(ex["task_dep"][c])):
            assert end[p] <= start[c], (p, c)
    # the same records as a Perfetto (trace-event) document: one slice per task
    # on its worker's track, the tracks' slices disjoint
    from task_graph_runtime_amd import trace_export
    doc = trace_export.chrome_trace(rec, tpu, ex, flows=True)
    tasks = [e for e in doc["traceEvents"] if e["ph"] == "X" and e["cat"] not in ("wait", "trigger", "phase")]
    assert sorted(e["args"]["task"] for e in tasks) == real.tolist()
    by_w = {}
    for e in tasks:
        by_w.setdefault(e["tid"], []).append((e["ts"], e["ts"] + e["dur"]))
    for sl in by_w.values():
        sl.sort()
        assert all(a[1] <= b[0] + 1e-6 for a, b in zip(sl, sl[1:]))
    r.g.set_trace(False)


# ------------------------------------------------------------------ region completeness
def reverse_priority_order(ex):
    """A topological order of the built graph that always runs, among the
    ready tasks, the one latest in program order (empty tasks resolve at
    once).  A task then runs before every task it does not wait for through
    the graph, so if its declared inputs miss a region some earlier task
    writes, it runs before that writer and reads the poison."""
    import heapq
    dep, trig, cnt = ex["task_dep"], ex["task_trig"], ex["event_counts"]
    first, last, orig, tt = ex["event_first"], ex["event_last"], ex["task_orig"], ex["task_type"]
    arrived = np.zeros(len(cnt), np.int64)
    heap, order = [], []

    def fire(e):
        for t in range(int(first[e]), int(last[e]) + 1):
            if tt[t] == mpk._binding.TASK_EMPTY:
                arrive(int(trig[t]))
            else:
                heapq.heappush(heap, (-int(orig[t]), t))

    def arrive(e):
        arrived[e] += 1
        if arrived[e] == cnt[e]:
            fire(e)
    fire(int(ex["header"]["root"]))
    while heap:
        _, t = heapq.heappop(heap)
        order.append(t)
        arrive(int(trig[t]))
    assert len(order) == int(np.sum(tt != mpk._binding.TASK_EMPTY))
    return order


@pytest.mark.parametrize("B,params", [(1, {}), (3, {}), (3, dict(k_qkv=3, k_o=2, k_down=4)),
                                      (2, dict(attn_jit=1))])
def test_regions_complete_serial_poisoned(B, params):
    """Every region a task reads is declared: with all activations NaN, the
    tasks run one at a time in the reverse-priority order above and the step
    still matches the oracle (a missing region would be read before its
    writer ran)."""
    s = TINY.with_(batch=B, ctx_range=(3, 120), ctx=0)
    say("regions complete", B, params)
    inp = device_inputs(s, seed=61 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    r = Runner(inp, params)
    r.run("mega")                       # sets the step's arguments
    order = reverse_priority_order(r.g.export())
    r.logits.fill_(float("nan"))
    r.next.fill_(-1)
    r.g.run_tasks(order, poison=True)
    torch.cuda.synchronize()
    check(r.logits.cpu().numpy(), r.next.cpu().numpy(), ref, ref_next)
    check_cache(inp, cap)


def test_serial_order_catches_a_missing_region():
    """The check above is not vacuous: the same serial run in the order that
    puts the O-projection tiles of layer 0 ahead of the attention splits they
    read (as a graph missing those regions would allow) produces NaN."""
    inp = device_inputs(TINY, seed=3)
    r = Runner(inp)
    r.run("mega")
    ex = r.g.export()
    order = reverse_priority_order(ex)
    tt, layer = ex["task_type"], ex["task_layer"]
    o0 = [t for t in order if tt[t] == mpk._binding.TASK_OPROJ and layer[t] == 0]
    a0 = [t for t in order if tt[t] == mpk._binding.TASK_ATTN and layer[t] == 0]
    rest = [t for t in order if t not in o0]
    k = rest.index(a0[0])
    r.g.run_tasks(rest[:k] + o0 + rest[k:], poison=True)
    torch.cuda.synchronize()
    assert np.isnan(r.logits.cpu().numpy()).all()


# ------------------------------------------------------------------ shapes off the beaten path
@pytest.mark.parametrize("B", [1, 3])
def test_tiny_head_dim_64_with_qk_norm(B):
    s = TINY.with_(qk_norm=True, batch=B, ctx_range=(3, 200), ctx=0)
    say("tiny d=64 qk_norm", B)
    inp = device_inputs(s, seed=71 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    for mode in ("mega", "base"):
        logits, nxt = Runner(inp).run(mode)
        check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.parametrize("B", [1, 3, 16])
def test_tiny_peaked_attention(B):
    """Cached keys scaled by 32 (exact in bf16): the scores spread over
    hundreds, so the running maximum of the online softmax rises many times
    within a split -- at batch > 1 every rise past the kernel's margin takes
    its rescale branch -- and most weights underflow to zero."""
    s = TINY.with_(batch=B, ctx_range=(120, 250), ctx=0)
    say("tiny peaked attention", B)
    inp = device_inputs(s, seed=91 + B)
    inp["kv"]["k_pool"].mul_(32)
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    for mode in ("mega", "base"):
        logits, nxt = Runner(inp).run(mode)
        check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.parametrize("P", [16, 32, 64])
@pytest.mark.parametrize("B", [1, 3])
def test_tiny_page_sizes(P, B):
    """Every page size the library takes (16, 32, 64 tokens) with ragged
    lengths that end inside, and exactly at the end of, a page."""
    s = TINY.with_(page_size=P, batch=B, ctx_range=(P - 1, 230), ctx=0)
    say("tiny page size", P, B)
    lens = [P - 1, 2 * P, 229][:B] if B > 1 else [3 * P - 1]
    inp = device_inputs(s, seed=141 + P + B, gamma="uniform", seq_lens=lens)
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    for mode in ("mega", "base"):
        logits, nxt = Runner(inp).run(mode)
        check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B", [1, 3, 16])
def test_largest_hidden(B):
    """The largest hidden size the kernels take (8192: the batch-1 tiles'
    staging registers full) with 64 query heads and FFN 24576, two layers: at
    batch 1 the pre-load shrinks to 8 segments per wavefront behind a 96 KB
    staging area, at batch 3 and 16 the default k-splits shrink to fit the
    norm tasks' staging in LDS."""
    s = TINY.with_(hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, ffn=24576, batch=B, ctx_range=(30, 200),
                   ctx=0)
    say("largest hidden", B)
    inp = device_inputs(s, seed=131 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    r = Runner(inp)
    for mode in ("mega", "base"):
        logits, nxt = r.run(mode)
        check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)
    del r
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,H,F", [(1, 264, 712), (1, 520, 1000), (3, 288, 352), (5, 320, 416)])
def test_odd_widths(B, H, F):
    """Widths that are not multiples of the tile and k-step quanta: at batch 1
    multiples of 8 only (partial 512-element segments), above it multiples of
    32 but not 64 or 128 (odd k-step counts, uneven k-split ranges)."""
    s = TINY.with_(hidden=H, ffn=F, batch=B, ctx_range=(3, 150), ctx=0)
    say("odd widths", B, H, F)
    inp = device_inputs(s, seed=81 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    for mode in ("mega", "base"):
        logits, nxt = Runner(inp).run(mode)
        check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


@pytest.mark.timeout(600)
def test_qwen3_8b_batch16_alternating_inputs():
    """Four steps of the 8B batch-16 graph alternating two token sets, each
    step against its own oracle: the matrix-core tiles read task-to-task
    inputs through the L2, so nothing of the previous step may survive there."""
    s = synth.SHAPES["qwen3_8b_b16"]
    say("8B b16 alternating", "generate")
    inp = device_inputs(s, seed=5)
    ids = [inp["token_ids"].clone(), (inp["token_ids"] * 7 + 13) % s.vocab]
    refs = []
    for k, t in enumerate(ids):
        say("8B b16 alternating", "oracle", k)
        inp["token_ids"] = t
        refs.append(run_oracle(inp, lazy=True, widen_on_device=True))
    r = Runner(inp)
    for i, k in enumerate([0, 1, 0, 1]):
        say("8B b16 alternating", "step", i, "tokens", k)
        r.inp["token_ids_dev"].copy_(ids[k].to(r.inp["token_ids_dev"].dtype).cuda())
        logits, nxt = r.run("mega")
        check(logits, nxt, *refs[k])
    del r
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,attn_jit", [(1, 0), (1, 1), (3, 0), (3, 1)])
def test_tiny_without_fusion(B, attn_jit):
    """The graph built without event fusion (one event per overlap edge,
    fan-in and fan-out rewrites, empty tasks two deep) runs to the same
    result; with attention JIT the fan-in events hand their splits over."""
    s = TINY.with_(batch=B, ctx_range=(3, 120), ctx=0)
    say("tiny no fusion", B, attn_jit)
    inp = device_inputs(s, seed=91 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    params = dict(n_workers=8, quantum=64 if B == 1 else 16, t_qkv=8, t_o=4, t_gu=11, t_down=4, t_lm=16, s_attn=4,
                  fusion_order=1, attn_jit=attn_jit)
    r = Runner(inp, params)
    assert r.g.header()["params"]["fusion_order"] == 1
    logits, nxt = r.run("mega")
    check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)


# ------------------------------------------------------------------ prepared weights (matrix-core load order)
@pytest.mark.parametrize("B,params", [(3, {}), (3, dict(k_qkv=3, k_o=2, k_down=4)), (16, {}), (5, dict(attn_jit=1))])
def test_prepared_weights(B, params):
    """mpk_prepare_weights copies every projection into 16 x 32 blocks in the
    matrix-core tile's lane order (gate/up interleaved); the step on the
    prepared copy matches the oracle and the step on the original weights."""
    s = TINY.with_(qk_norm=True, batch=B, ctx_range=(3, 200), ctx=0)
    say("prepared weights", B, params)
    inp = device_inputs(s, seed=111 + B, gamma="uniform")
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    r = Runner(inp, params)
    plain, plain_next = r.run("mega")
    check(plain, plain_next, ref, ref_next)
    pw = mpk.PreparedWeights(r.g, r.w)
    assert pw.s.layout == 1
    r.w = pw
    for mode in ("mega", "base"):
        logits, nxt = r.run(mode)
        check(logits, nxt, ref, ref_next)
        np.testing.assert_allclose(logits, plain, rtol=1e-4, atol=1e-4)
    check_cache(inp, cap)


def test_prepared_weights_refused_at_batch_one():
    inp = device_inputs(TINY, seed=120)
    r = Runner(inp)
    with pytest.raises(mpk.MpkError) as e:
        mpk.PreparedWeights(r.g, r.w)
    assert e.value.code == -2


@pytest.mark.timeout(600)
def test_qwen3_8b_batch16_prepared_weights():
    s = synth.SHAPES["qwen3_8b_b16"]
    say("8B b16 prepared", "generate")
    inp = device_inputs(s, seed=0)
    say("8B b16 prepared", "oracle")
    ref, ref_next = run_oracle(inp, lazy=True, widen_on_device=True)
    r = Runner(inp)
    r.run("mega")
    r.w = mpk.PreparedWeights(r.g, r.w)
    say("8B b16 prepared", "mega")
    logits, nxt = r.run("mega")
    say("8B b16 prepared", "max |d|", check(logits, nxt, ref, ref_next))
    del r
    torch.cuda.empty_cache()
