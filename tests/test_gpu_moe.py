"""GPU parity of mixture-of-experts decode steps (the Qwen3-MoE reading of
the MoE layer) through the C ABI against the oracle.

Routing is an integer decision taken from floating-point router logits.
Where the oracle's k-th and (k+1)-th expert probabilities are more than TAU
apart, the kernel must choose exactly the oracle's experts.  Closer than that
(a near-tie: either set is correct up to rounding) the kernel's set must be a
valid top-k within TAU, and the oracle then follows the kernel's choice
(its route hook), so that the rest of the step is compared like for like.
The route records also fix the slot order: slot s serves the s-th smallest
chosen expert, idle slots (expert -1) last, tokens ascending in each slot.
"""
import numpy as np
import pytest
import torch

import synth
import task_graph_runtime_amd as mpk
from oracle import numerics as on
from tests._util import run_oracle
from tests.test_gpu_decode import Runner, check, check_cache, device_inputs, reverse_priority_order, say

pytestmark = pytest.mark.gpu

TAU = 1e-4          # probability gap below which a routing choice is a near-tie
W_ATOL = 2e-3       # expert weights (probabilities renormalised over the chosen experts)
TINY_MOE = synth.SHAPES["tiny_moe"]


def tensor_id(l, k):
    return 5 + mpk._binding.LAYER_TENSORS * l + k


def gpu_routes(g, s):
    """Per layer: {request: {expert: weight}} from the route records, after
    checking their form."""
    B, k = s.batch, s.top_k
    M, rw = min(s.n_experts, B * k), 2 + 2 * B
    out = []
    for l in range(s.n_layers):
        rec = g.read_tensor(tensor_id(l, 14), (M, rw), np.int32)
        routes = {b: {} for b in range(B)}
        busy = []
        for r in rec:
            e, n = int(r[0]), int(r[1])
            if e < 0:
                assert n == 0, r
                continue
            assert 0 < n <= B and e < s.n_experts, r
            busy.append(e)
            toks = [int(x) for x in r[2:2 + n]]
            assert toks == sorted(set(toks)) and all(0 <= b < B for b in toks), r
            for b, w in zip(toks, r[2 + B:2 + B + n].view(np.float32)):
                routes[b][e] = float(w)
        experts = [int(r[0]) for r in rec]
        nb = len(busy)
        assert busy == sorted(busy) and len(set(busy)) == nb, experts
        assert experts[nb:] == [-1] * (M - nb), experts
        for b in range(B):
            assert len(routes[b]) == k, (l, b, routes[b])
        out.append(routes)
    return out


class FollowNearTies:
    """Route hook for the oracle: the kernel's experts must equal the
    oracle's where the choice is clear, and be a valid top-k within TAU at a
    near-tie, where the oracle takes them."""

    def __init__(self, routes, k):
        self.routes, self.k = routes, k
        self.ties = 0

    def __call__(self, l, logits, ids, margin):
        p = on.softmax(np.asarray(logits, dtype=np.float64))
        forced = ids.copy()
        for b in range(ids.shape[0]):
            got, want = set(self.routes[l][b]), set(int(e) for e in ids[b])
            if margin[b] > TAU:
                assert got == want, (l, b, sorted(got), sorted(want), float(margin[b]))
                continue
            kth = np.sort(p[b])[::-1][self.k - 1]
            assert all(p[b, e] >= kth - TAU for e in got), (l, b, sorted(got), sorted(want))
            if got != want:
                self.ties += 1
                forced[b] = sorted(got, key=lambda e: (-p[b, e], e))
        return forced


def check_moe_step(r, inp, logits, nxt, intermediates=True):
    """Routes, weights, the layer outputs and the step against the oracle."""
    s = inp["shape"]
    routes = gpu_routes(r.g, s)
    hook = FollowNearTies(routes, s.top_k)
    cap = {}
    lazy = s.n_layers * s.n_experts * s.moe_ffn * s.hidden > 50_000_000
    ref, ref_next = run_oracle(inp, capture=cap, lazy=lazy, route_hook=hook)
    say(s.name, "B", s.batch, "near-ties followed:", hook.ties)
    for l in range(s.n_layers):
        c = cap[l]
        for b in range(s.batch):
            w_gpu = np.array([routes[l][b][int(e)] for e in c["expert_ids"][b]])
            np.testing.assert_allclose(w_gpu, c["expert_weights"][b], atol=W_ATOL, err_msg=f"weights l={l} b={b}")
            if s.norm_topk:
                assert abs(w_gpu.sum() - 1.0) < 1e-5
        if intermediates:
            B, H, E = s.batch, s.hidden, s.n_experts
            np.testing.assert_allclose(r.g.read_tensor(tensor_id(l, 13), (B, E), np.float32), c["router_logits"],
                                       rtol=3e-2, atol=3e-2, err_msg=f"router logits l={l}")
            np.testing.assert_allclose(r.g.read_tensor(tensor_id(l, 10), (B, H), np.float32), c["h2"],
                                       rtol=3e-2, atol=3e-2, err_msg=f"h2 l={l}")
            np.testing.assert_allclose(r.g.read_tensor(tensor_id(l, 12), (B, H), np.float32), c["d"],
                                       rtol=3e-2, atol=3e-2, err_msg=f"d l={l}")
    err = check(logits, nxt, ref, ref_next)
    check_cache(inp, cap)
    return err


def moe_shape(B, **kw):
    s = TINY_MOE.with_(batch=B, **kw)
    return s if B == 1 else s.with_(ctx_range=(3, 120), ctx=0)


@pytest.mark.parametrize("B", [1, 3, 16])
@pytest.mark.parametrize("mode", ["mega", "base", "graph"])
def test_tiny_moe(B, mode):
    say("tiny_moe", B, mode)
    inp = device_inputs(moe_shape(B), seed=11 + B, gamma="uniform")
    r = Runner(inp)
    logits, nxt = r.run(mode)
    check_moe_step(r, inp, logits, nxt)


@pytest.mark.parametrize("B", [1, 5])
@pytest.mark.parametrize("params", [dict(attn_jit=1), dict(attn_jit=3), dict(weight_preload=2),
                                    dict(fusion_order=1), dict(t_router=1, t_egu=1, t_edown=1),
                                    dict(t_router=1, t_egu=3, t_edown=5)])
def test_tiny_moe_build_params(B, params):
    say("tiny_moe params", B, params)
    inp = device_inputs(moe_shape(B), seed=23 + B, gamma="uniform")
    r = Runner(inp, params)
    logits, nxt = r.run("mega")
    check_moe_step(r, inp, logits, nxt, intermediates=False)


@pytest.mark.parametrize("B,kw", [(1, dict(top_k=1)), (3, dict(top_k=1)), (2, dict(top_k=8)),
                                  (3, dict(norm_topk=0)), (16, dict(n_experts=256, top_k=16, moe_ffn=64)),
                                  (1, dict(n_experts=200, top_k=5))])
def test_tiny_moe_routing_shapes(B, kw):
    """One expert per token; every expert chosen (k = E: no tie possible);
    weights not renormalised; 256 experts, 16 per token (every slot of the
    batch, the largest route); an expert count that is not a multiple of 64."""
    say("tiny_moe routing", B, kw)
    inp = device_inputs(moe_shape(B, **kw), seed=31 + B, gamma="uniform")
    r = Runner(inp)
    logits, nxt = r.run("mega")
    check_moe_step(r, inp, logits, nxt)


@pytest.mark.parametrize("B,zero", [(1, range(8)), (3, range(8)), (1, range(4, 8)), (3, range(4, 8)),
                                    (16, range(2, 8, 2))])
def test_tiny_moe_exact_ties(B, zero):
    """Router rows of some experts set to zero: their logits are exactly 0 for
    every token, so the choice between them is an exact tie, which goes to the
    lowest index (all rows zero: experts 0..k-1 with weight 1/k each).  Here
    the kernel's sets must equal the oracle's exactly, whatever the margin."""
    say("tiny_moe ties", B, list(zero))
    inp = device_inputs(moe_shape(B), seed=71 + B, gamma="uniform")
    for lw in inp["weights"]["layers"]:
        lw["router"][list(zero)] = 0
    r = Runner(inp)
    logits, nxt = r.run("mega")
    routes = gpu_routes(r.g, inp["shape"])
    cap = {}
    ref, ref_next = run_oracle(inp, capture=cap)
    k = inp["shape"].top_k
    for l in range(inp["shape"].n_layers):
        for b in range(B):
            want = [int(e) for e in cap[l]["expert_ids"][b]]
            assert set(routes[l][b]) == set(want), (l, b, routes[l][b], want)
            np.testing.assert_allclose([routes[l][b][e] for e in want], cap[l]["expert_weights"][b], atol=W_ATOL)
            if len(zero) == 8:
                assert sorted(routes[l][b]) == list(range(k))
                np.testing.assert_allclose(list(routes[l][b].values()), 1.0 / k, rtol=1e-6)
    check(logits, nxt, ref, ref_next)


def test_tiny_moe_consecutive_steps():
    """Three steps on one graph with different inputs each: the layer outputs
    that the experts add into start every step at zero."""
    s = moe_shape(3)
    r = None
    for seed in (41, 42, 43):
        say("tiny_moe consecutive", seed)
        inp = device_inputs(s, seed=seed, gamma="uniform")
        if r is None:
            r = Runner(inp)
        else:
            r.inp = inp
            kv = inp["kv"]
            r.w = mpk.Weights(inp["weights"])
            r.kv = mpk.KV(kv["k_pool"], kv["v_pool"], kv["page_table_dev"])
        logits, nxt = r.run("mega")
        check_moe_step(r, inp, logits, nxt, intermediates=False)


@pytest.mark.parametrize("B,params", [(1, {}), (3, {}), (2, dict(attn_jit=1))])
def test_tiny_moe_regions_complete_serial_poisoned(B, params):
    """Every region an expert task reads is declared: all activations NaN,
    the tasks run one at a time in reverse-priority order, and the step still
    matches the oracle."""
    say("tiny_moe regions complete", B, params)
    inp = device_inputs(moe_shape(B), seed=51 + B, gamma="uniform")
    r = Runner(inp, params)
    r.run("mega")
    order = reverse_priority_order(r.g.export())
    r.logits.fill_(float("nan"))
    r.next.fill_(-1)
    r.g.run_tasks(order, poison=True)
    torch.cuda.synchronize()
    check_moe_step(r, inp, r.logits.cpu().numpy(), r.next.cpu().numpy(), intermediates=False)


def _full(name, modes, builds=()):
    s = synth.SHAPES[name]
    say(name, "inputs")
    inp = device_inputs(s, seed=0)
    for params in ({},) + tuple(builds):
        for mode in (modes if not params else ("mega",)):
            say(name, mode, params)
            r = Runner(inp, params)
            logits, nxt = r.run(mode)
            err = check_moe_step(r, inp, logits, nxt, intermediates=False)
            say(name, mode, params, "max |d|", err)
            del r
    del inp
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_qwen3_30b_a3b_shape():
    _full("qwen3_30b_a3b", modes=("mega", "base"))


@pytest.mark.timeout(900)
def test_qwen3_30b_a3b_batch16_shape():
    _full("qwen3_30b_a3b_b16", modes=("mega",), builds=(dict(attn_jit=1),))
