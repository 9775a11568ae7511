"""The no-allocation decode step (mpk_decode_step_noalloc) against the step
it is a variant of (mpk_decode_step) and against the oracle: two calls in a
row on two graphs, the second with a smaller input, then the first graph
again; plus the refusal of a graph whose state exceeds the static area."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
import task_graph_runtime_amd as mpk
from oracle import numerics as on
from tests._util import run_oracle
from tests.test_gpu_decode import ATOL, RTOL, GAP, Runner, check, check_cache, device_inputs, say

pytestmark = pytest.mark.gpu

TINY = synth.SHAPES["tiny"]


def noalloc(r):
    r.logits.fill_(float("nan"))
    r.next.fill_(-1)
    r.g.decode_step_noalloc(r.w, r.inp["token_ids_dev"], r.kv, r.inp["seq_lens_dev"], r.logits, r.next)
    torch.cuda.synchronize()
    assert r.g.status()["code"] == 0
    return r.logits.cpu().numpy(), r.next.cpu().numpy()


def against(got, got_next, ref, ref_next):
    """got within the logits bound of ref, ids equal where ref's top-2 gap exceeds it."""
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)) and not np.any(err > ATOL + RTOL * np.abs(ref)), float(err.max())
    m = on.top2_gap(ref) > GAP
    assert np.array_equal(got_next[m], ref_next[m])


def test_noalloc_matches_the_regular_step_on_two_graphs():
    sa = TINY.with_(batch=3, ctx_range=(20, 200), ctx=0)
    sb = TINY.with_(batch=1, ctx=40)                     # the second call: a smaller input
    runs = []
    for s, seed in ((sa, 101), (sb, 102)):
        inp = device_inputs(s, seed=seed, gamma="uniform")
        cap = {}
        ref = run_oracle(inp, capture=cap)
        r = Runner(inp)
        runs.append((r, ref, cap, inp))
    for k, (r, ref, cap, inp) in enumerate(runs + runs[:1]):
        say("noalloc call", k, "batch", inp["shape"].batch)
        logits, nxt = r.run("mega")                      # the regular step (binds the weights)
        check(logits, nxt, *ref)
        got, got_next = noalloc(r)
        against(got, got_next, logits, nxt)              # against the step it is a variant of
        check(got, got_next, *ref)                       # and against the oracle
        check_cache(inp, cap)


def test_noalloc_requires_bound_weights_and_a_fitting_graph():
    inp = device_inputs(TINY, seed=103)
    r = Runner(inp)
    with pytest.raises(mpk.MpkError) as e:                # no regular step yet: weights unbound
        noalloc(r)
    assert e.value.code == -1 and "not bound" in str(e.value)
    # the 8B batch-16 graph keeps ~150 MB of activations: more than the static area
    s = synth.SHAPES["qwen3_8b_b16"]
    g = mpk.TGraph(s.cfg(), s.batch, s.page_size)
    rc = mpk.lib().mpk_decode_step_noalloc(g.h, C.byref(r.w.s), C.c_void_p(1), C.byref(r.kv.s), C.c_void_p(1),
                                           C.c_void_p(1), C.c_void_p(1), None)
    assert rc == -2 and "static area" in mpk.lib().mpk_last_error().decode()
    g.close()
