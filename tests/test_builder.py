"""The C++ tGraph builder (through the C ABI, host only) against the oracle spec,
bit for bit on every exported index array, plus the C ABI surface (CPU only)."""
import ctypes as C
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, HealthCheck

import synth
import task_graph_runtime_amd as mpk
from oracle import tgraph as tg
from tests.test_tgraph_oracle import programs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ARRAYS = ["task_type", "task_mode", "task_layer", "task_coords", "task_orig", "task_dep", "task_trig",
          "task_worker", "event_counts", "event_first", "event_last", "event_flags", "aot_offsets", "aot_tasks"]


def assert_same(ref, got):
    for k in ARRAYS:
        assert ref[k].dtype == got[k].dtype, k
        assert np.array_equal(ref[k], got[k]), k
    assert ref["header"] == got["header"]


def both(shape, B, W, q=None, S=None, **over):
    """Build the same graph with the C++ builder (defaults resolved by the
    library, overrides applied) and with the oracle spec (params read back
    from the library's header)."""
    s = shape
    names = dict(T_qkv="t_qkv", T_o="t_o", T_gu="t_gu", T_down="t_down", T_lm="t_lm", K_qkv="k_qkv", K_o="k_o",
                 K_down="k_down", coarse="coarse_events", fusion="fusion_order", T_router="t_router", T_egu="t_egu",
                 T_edown="t_edown")
    params = dict(n_workers=W, s_attn=S or max(4, B), attn_jit=over.pop("attn_jit", 0))
    if q is not None:
        params["quantum"] = q
    for k, v in over.items():
        params[names[k]] = v
    g = mpk.TGraph(s.cfg(), B, s.page_size, params, host_only=True)
    p = g.header()["params"]
    prm = tg.Params(W=p["n_workers"], S_sched=p["n_sched_waves"], q=p["quantum"], T_qkv=p["t_qkv"], T_o=p["t_o"],
                    T_gu=p["t_gu"], T_down=p["t_down"], T_lm=p["t_lm"], S_attn=p["s_attn"],
                    jit_attn=p["attn_jit"] == 1, jit_all=p["attn_jit"] == 3, K_qkv=p["k_qkv"], K_o=p["k_o"],
                    K_down=p["k_down"], coarse=p["coarse_events"] == 1, fusion=p["fusion_order"],
                    T_router=p["t_router"] or 1, T_egu=p["t_egu"] or 1, T_edown=p["t_edown"] or 1)
    ref, tasks = tg.build(s.cfg(), B, s.page_size, prm)
    got = g.export()
    got["params"] = p
    return ref, got, tasks


@pytest.mark.parametrize("attn_jit", [0, 1, 2])
def test_tiny_worked_example_bit_exact(attn_jit):
    s = synth.SHAPES["tiny"]
    ref, got, tasks = both(s, 1, 8, q=64, S=4, T_qkv=8, T_o=4, T_gu=11, T_down=4, T_lm=16, attn_jit=attn_jit)
    assert_same(ref, got)
    assert got["header"]["NT"] == 95 and got["header"]["NE"] == 19
    # default at batch 1: attention AOT
    assert got["params"]["attn_jit"] == (1 if attn_jit == 1 else 2)
    n_jit = int(np.sum(got["task_mode"] == tg.MODE_JIT))
    assert n_jit == (16 if attn_jit == 1 else 0)
    tg.check_semantics(got, tasks, closure=True)


@pytest.mark.parametrize("B,attn_jit,resolved", [(2, 0, 2), (2, 1, 1), (2, 2, 2), (16, 0, 2), (16, 1, 1), (1, 3, 3),
                                                  (3, 3, 3)])
def test_attention_policy_at_batch_above_one(B, attn_jit, resolved):
    s = synth.SHAPES["tiny"].with_(n_layers=1)
    ref, got, tasks = both(s, B, 13, S=max(2, B), attn_jit=attn_jit)
    assert_same(ref, got)
    assert got["params"]["attn_jit"] == resolved
    tg.check_semantics(got, tasks, closure=True)


@pytest.mark.parametrize("K", [(1, 1, 1), (3, 2, 4), (2, 5, 3)])
def test_k_split_bit_exact(K):
    """Projections split along their contraction (batch > 1): tile n is column
    tile n / K over k range n % K, its output one of K planes that the
    consumers read whole."""
    s = synth.SHAPES["tiny"]
    ref, got, tasks = both(s, 3, 13, S=4, K_qkv=K[0], K_o=K[1], K_down=K[2])
    assert_same(ref, got)
    p = got["params"]
    assert (p["k_qkv"], p["k_o"], p["k_down"]) == K
    assert p["t_qkv"] % (s.n_kv_heads * K[0]) == 0 and p["t_o"] % K[1] == 0 and p["t_down"] % K[2] == 0
    tg.check_semantics(got, tasks, closure=True)


def test_all_jit_policy():
    """attn_jit = 3: every non-empty task JIT but the root's consumers (nothing
    triggers the root event, so nothing would hand them over), so schedulers
    exist at batch 1 too."""
    s = synth.SHAPES["tiny"]
    ref, got, tasks = both(s, 1, 12, S=4, attn_jit=3)
    assert_same(ref, got)
    md, tt, dep = got["task_mode"], got["task_type"], got["task_dep"]
    root = got["header"]["root"]
    assert np.all(md[(tt != tg.EMPTY) & (dep != root)] == tg.MODE_JIT)
    assert np.all(md[dep == root] == tg.MODE_AOT) and got["aot_offsets"][-1] == np.sum(dep == root)
    assert np.all(tt[dep == root] == tg.QKV)   # the layer-0 projection tiles (batch 1)
    assert got["params"]["n_sched_waves"] > 0
    tg.check_semantics(got, tasks, closure=True)


@pytest.mark.parametrize("B", [1, 3])
def test_coarse_operator_level_graph(B):
    """coarse_events = 1, the operator-level graph: every task waits for the
    whole previous operator, so all tiles of one operator (one layer and task
    type) share one dependent event -- also the k-split O and down tiles at
    batch > 1, which the fine graph lets wait for their own k-range only."""
    s = synth.SHAPES["tiny"]
    ref, got, tasks = both(s, B, 13, S=4, coarse=1)
    assert_same(ref, got)
    tg.check_semantics(got, tasks, closure=True)
    _, fine, _ = both(s, B, 13, S=4)
    if B > 1:   # (the tiny shape's 2 kv groups: 2 O ranges)
        assert got["params"]["k_o"] == 2 and got["params"]["k_down"] == 3

    def deps(g, ty):
        real = g["task_type"] == ty
        return {(int(l), int(d)) for l, d in zip(g["task_layer"][real], g["task_dep"][real])}
    for ty in (tg.QKV, tg.ATTN, tg.OPROJ, tg.GATEUP, tg.DOWN, tg.LMHEAD):
        d = deps(got, ty)
        assert len(d) == len({l for l, _ in d}), tg.TYPE_NAMES[ty]   # one event per operator
    att = lambda g: set(g["task_dep"][g["task_type"] == tg.ATTN].tolist())
    assert len(att(got)) == s.n_layers and len(att(fine)) == s.n_layers * s.n_kv_heads
    if B > 1:   # fine: the O and down tiles wait per k-range
        assert len(deps(fine, tg.OPROJ)) == 2 * s.n_layers and len(deps(fine, tg.DOWN)) == 3 * s.n_layers


def test_weight_preload_switch():
    s = synth.SHAPES["tiny"]
    for v, want in ((0, 1), (1, 1), (2, 2), (3, 3)):
        p = mpk.TGraph(s.cfg(), 1, s.page_size, dict(weight_preload=v), host_only=True).header()["params"]
        assert p["weight_preload"] == want
    with pytest.raises(mpk.MpkError):
        mpk.TGraph(s.cfg(), 1, s.page_size, dict(weight_preload=4), host_only=True)


def test_k_split_default_yields_to_a_given_tile_count():
    s = synth.SHAPES["tiny"]
    # (2 kv groups: the O default is 2 ranges, kept by t_o = 4, dropped by t_o = 5; down 3, kept by 6)
    p = mpk.TGraph(s.cfg(), 3, s.page_size, dict(n_workers=13, s_attn=4, t_o=4, t_down=6), host_only=True)
    p = p.header()["params"]
    assert (p["k_o"], p["k_down"], p["t_o"], p["t_down"]) == (2, 3, 4, 6)
    p = mpk.TGraph(s.cfg(), 3, s.page_size, dict(n_workers=13, s_attn=4, t_o=5, t_down=4), host_only=True)
    p = p.header()["params"]
    assert (p["k_o"], p["k_down"], p["t_o"], p["t_down"]) == (1, 1, 5, 4)


@pytest.mark.parametrize("B,over", [(1, dict(k_qkv=2)), (1, dict(k_down=2)), (2, dict(k_o=1000)),
                                    (2, dict(k_qkv=2, t_qkv=6))])
def test_bad_k_split_rejected(B, over):
    s = synth.SHAPES["tiny"]
    with pytest.raises(mpk.MpkError):
        mpk.TGraph(s.cfg(), B, s.page_size, dict(n_workers=13, s_attn=4) | over, host_only=True)


@pytest.mark.parametrize("name,B,W,S,layers", [
    ("tiny", 1, 8, 4, 2), ("tiny", 5, 13, 7, 2), ("tiny", 16, 252, 20, 2),
    ("qwen3_0p6b", 1, 252, 16, 2), ("qwen3_8b", 1, 252, 16, 1), ("qwen3_8b_b16", 16, 252, 31, 1),
    ("qwen3_32b", 1, 252, 16, 1)])
def test_layer_cuts_bit_exact(name, B, W, S, layers):
    s = synth.SHAPES[name].with_(n_layers=layers)
    ref, got, tasks = both(s, B, W, S=S)
    assert_same(ref, got)
    tg.check_semantics(got, tasks, closure=(len(tasks) < 3000))


@pytest.mark.parametrize("name", ["qwen3_0p6b", "qwen3_8b", "qwen3_8b_b16"])
def test_full_graph_bit_exact(name):
    s = synth.SHAPES[name]
    ref, got, _ = both(s, s.batch, 252, S=16 if s.batch == 1 else 31)
    assert_same(ref, got)
    tg.check_semantics(got, None)


def test_default_params_resolve_as_documented():
    s = synth.SHAPES["qwen3_8b"]
    h = mpk.TGraph(s.cfg(), 1, 64, {}, host_only=True).header()
    p = h["params"]
    # batch 1: attention is AOT, nothing is JIT, so no scheduler workgroups: 256 workers
    assert p["n_workers"] == 256 and p["n_sched_waves"] == 0 and p["quantum"] == 1 and p["attn_jit"] == 2
    # one attention task per worker: 256 / 8 = 32 slots per kv group (the step uses as many as the
    # cached length and the combine's staging allow); at least one page per split
    assert p["t_qkv"] == 256 and p["t_o"] == p["t_gu"] == p["t_down"] == p["t_lm"] == 256 and p["s_attn"] == 32
    assert p["attn_split_pages"] == 1
    h16 = mpk.TGraph(s.cfg(), 16, 64, {}, host_only=True).header()["params"]
    # batch 16: every task AOT by default too, so no scheduler workgroups: 256 workers
    assert h16["n_workers"] == 256 and h16["n_sched_waves"] == 0 and h16["attn_jit"] == 2
    # one attention task per worker: 256 / 8 = 32 slots per kv group, dealt to the 16 requests by pages
    assert h16["quantum"] == 16 and h16["s_attn"] == 32
    # 151936 columns x 16 requests need >= 297 tiles of <= 8192 accumulators: two per worker
    assert h16["t_lm"] == 512 and h16["t_gu"] == 256
    # the output projection splits its contraction into 4 ranges of 2 kv groups (64 column tiles x 4),
    # the down projection 3 ways (85 column tiles x 3)
    assert (h16["k_qkv"], h16["k_o"], h16["k_down"]) == (1, 4, 3)
    assert h16["t_qkv"] == 256 and h16["t_o"] == 256 and h16["t_down"] == 255
    # the hybrid policy (attention JIT): 14 scheduler wavefronts (4 workgroups) leave 252 workers
    hj = mpk.TGraph(s.cfg(), 16, 64, dict(attn_jit=1), host_only=True).header()["params"]
    assert hj["n_workers"] == 252 and hj["n_sched_waves"] == 14 and hj["attn_jit"] == 1 and hj["s_attn"] == 31
    assert (p["k_qkv"], p["k_o"], p["k_down"]) == (1, 1, 1)


def test_default_k_splits_fit_the_norm_staging():
    """At batch > 1 a norm task stages the gain (bf16), the residual row and
    every k-split plane of its input (fp32) in LDS: at hidden 8192 the
    default splits (4 and 3) would need 176 KB, so they shrink until the
    staging takes at most 128 KB; the 8B and 32B shapes keep theirs, and
    splits given explicitly are kept."""
    kb = lambda b: (b + 1023) // 1024 * 1024
    big = synth.SHAPES["tiny"].with_(hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, ffn=24576)
    for B in (3, 16):
        p = mpk.TGraph(big.cfg(), B, big.page_size, {}, host_only=True).header()["params"]
        assert kb(8192 * 2) + (1 + max(p["k_o"], p["k_down"])) * kb(8192 * 4) <= 128 * 1024, p
        assert p["k_o"] >= 1 and 8 % p["k_o"] == 0 and p["k_down"] >= 1
        assert p["t_o"] % p["k_o"] == 0 and p["t_down"] % p["k_down"] == 0
    given = mpk.TGraph(big.cfg(), 3, big.page_size, dict(k_o=4, k_down=3), host_only=True).header()["params"]
    assert (given["k_o"], given["k_down"]) == (4, 3)
    for name, K in (("qwen3_8b", (4, 3)), ("qwen3_32b", (4, 3))):
        s = synth.SHAPES[name]
        p = mpk.TGraph(s.cfg(), 16, s.page_size, {}, host_only=True).header()["params"]
        assert (p["k_o"], p["k_down"]) == K, (name, p)


@settings(max_examples=120, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(programs())
def test_generic_entry_matches_spec(prog):
    specs, regions, W = prog
    tasks = tg.generic_tasks(specs, regions)
    ref = tg.canonicalize(tasks, W)
    got = mpk.build_generic(specs, regions, W)
    assert_same(ref, got)


@settings(max_examples=120, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(programs())
def test_generic_entry_without_fusion_matches_spec(prog):
    """The fan-in rewrite (no fusion) in the C++ builder against the spec, on
    random programs with misaligned tilings."""
    specs, regions, W = prog
    tasks = tg.generic_tasks(specs, regions)
    ref = tg.canonicalize(tasks, W, fusion=tg.FUSION_OFF)
    got = mpk.build_generic(specs, regions, W, fusion_order=1)
    assert_same(ref, got)


@pytest.mark.parametrize("B,attn_jit", [(1, 0), (1, 1), (3, 0), (3, 3)])
def test_decoder_without_fusion_bit_exact(B, attn_jit):
    s = synth.SHAPES["tiny"]
    ref, got, tasks = both(s, B, 8, q=64 if B == 1 else 16, S=4, T_qkv=8, T_o=4 if B == 1 else 6, T_gu=11,
                           T_down=4 if B == 1 else 6, T_lm=16, attn_jit=attn_jit, fusion=1)
    assert_same(ref, got)
    assert got["params"]["fusion_order"] == 1
    tg.check_semantics(got, tasks, closure=True)
    # the fan-in rewrite is in use: empties waiting on an event that another empty did not fire
    assert np.any(got["task_coords"][got["task_type"] == tg.EMPTY][:, 1] == 1)


# ------------------------------------------------------------------ C ABI surface
def header_symbols():
    text = open(os.path.join(ROOT, "include", "mpk.h")).read()
    return sorted(set(re.findall(r"\b(mpk_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = C.CDLL(os.path.join(ROOT, "task_graph_runtime_amd", "libmpk.so"))
    syms = header_symbols()
    assert len(syms) >= 13
    for name in syms:
        assert hasattr(L, name), name
    assert set(syms) == set(mpk.SIGNATURES)


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96), -2), (dict(n_q_heads=5), -1), (dict(hidden=260), -2), (dict(qk_norm=2), -1)])
def test_bad_config_rejected(over, code):
    c = mpk.model_cfg(synth.SHAPES["tiny"].cfg())
    for k, v in over.items():
        setattr(c, k, v)
    with pytest.raises(mpk.MpkError) as e:
        mpk.TGraph(c, 1, 16, {}, host_only=True)
    assert e.value.code == code


@pytest.mark.parametrize("B,P,params,code", [
    (0, 16, {}, -2), (17, 16, {}, -2), (1, 24, {}, -2), (1, 16, dict(t_qkv=3), -1),
    (1, 16, dict(fusion_order=2), -2), (1, 16, dict(t_o=100000), -1)])
def test_bad_build_args_rejected(B, P, params, code):
    with pytest.raises(mpk.MpkError) as e:
        mpk.TGraph(synth.SHAPES["tiny"].cfg(), B, P, params, host_only=True)
    assert e.value.code == code


def test_failed_build_clears_the_handle():
    """On every error, including a null config, *out is NULL afterwards."""
    h = C.c_void_p(0x1)
    p = mpk.mpk_build_params()
    p.host_only = 1
    assert mpk.lib().mpk_build_tgraph_ex(None, 1, 16, C.byref(p), C.byref(h)) == -1
    assert h.value is None
    h = C.c_void_p(0x1)
    c = mpk.model_cfg(synth.SHAPES["tiny"].cfg())
    c.head_dim = 96
    assert mpk.lib().mpk_build_tgraph_ex(C.byref(c), 1, 16, C.byref(p), C.byref(h)) == -2
    assert h.value is None


def test_reset_refuses_host_only_and_null():
    g = mpk.TGraph(synth.SHAPES["tiny"].cfg(), 1, 16, {}, host_only=True)
    assert mpk.lib().mpk_reset_tgraph(g.h) == -1
    assert mpk.lib().mpk_reset_tgraph(None) == -1


def test_host_only_graph_refuses_to_run():
    g = mpk.TGraph(synth.SHAPES["tiny"].cfg(), 1, 16, {}, host_only=True)
    w = mpk.mpk_weights()
    rc = mpk.lib().mpk_decode_step(g.h, C.byref(w), None, None, None, None, None, None)
    assert rc == -1


def test_generic_entry_rejects_bad_regions():
    with pytest.raises(mpk.MpkError):
        mpk.build_generic([(2, 0, 0, 0, 0)], [(5, 1, 0, (0, 0, 0, 0), (1, 1, 1, 1))], 1)


@pytest.mark.parametrize("over", [dict(hidden=264), dict(ffn=712), dict(hidden=264, ffn=712), dict(hidden=280)])
def test_partial_k_step_shapes_refused_above_batch_one(over):
    """Batch > 1 runs the projections on the matrix cores in whole 32-element
    contraction steps, with k-split ranges on 128-byte boundaries of the fp32
    rows: a hidden or ffn size that is a multiple of 8 but not of 32 is refused
    there (MPK_ERR_UNSUPPORTED) and still accepted at batch 1, whose tiles take
    the contraction 8 elements per lane."""
    c = mpk.model_cfg(synth.SHAPES["tiny"].cfg())
    for k, v in over.items():
        setattr(c, k, v)
    for B in (2, 3, 16):
        with pytest.raises(mpk.MpkError) as e:
            mpk.TGraph(c, B, 16, {}, host_only=True)
        assert e.value.code == -2 and "multiples of 32" in str(e.value)
    g = mpk.TGraph(c, 1, 16, {}, host_only=True)
    assert g.header()["n_tasks"] > 0


# ------------------------------------------------------------------ mixture of experts
@pytest.mark.parametrize("B,attn_jit,over", [(1, 0, dict(T_router=2, T_egu=3, T_edown=2)), (1, 1, {}),
                                              (3, 0, dict(T_egu=2, T_edown=2)), (4, 1, {}), (16, 0, {})])
def test_moe_graph_bit_exact(B, attn_jit, over):
    """Expert layers (router tiles, per-slot gate/up and down tiles) in the C++
    builder against the spec, with the closure check; a slot's down tiles wait
    for that slot's gate/up tiles only."""
    s = synth.SHAPES["tiny_moe"]
    ref, got, tasks = both(s, B, 8, q=1 if B == 1 else 16, S=max(4, B), attn_jit=attn_jit, **over)
    assert_same(ref, got)
    tg.check_semantics(got, tasks, closure=True)
    tt, dep = got["task_type"], got["task_dep"]
    M = min(s.n_experts, B * s.top_k)
    assert np.sum(tt == tg.EXPERT_GU) == s.n_layers * M * got["params"]["t_egu"]
    # one dependent event per slot (and layer) for the down tiles, one per layer for gate/up
    assert len(set(dep[tt == tg.EXPERT_DOWN].tolist())) == s.n_layers * M
    assert len(set(dep[tt == tg.EXPERT_GU].tolist())) == s.n_layers
    if attn_jit == 1:   # the hybrid policy makes the data-dependent tasks JIT: attention and experts
        assert np.all(got["task_mode"][np.isin(tt, (tg.ATTN, tg.EXPERT_GU, tg.EXPERT_DOWN))] == tg.MODE_JIT)


@pytest.mark.parametrize("name", ["qwen3_30b_a3b", "qwen3_30b_a3b_b16"])
def test_moe_full_graph(name):
    s = synth.SHAPES[name]
    g = mpk.TGraph(s.cfg(), s.batch, s.page_size, {}, host_only=True)
    p = g.header()["params"]
    ex = g.export()
    tg.check_semantics(ex, None)
    M = min(s.n_experts, s.batch * s.top_k)
    if s.batch == 1:
        # 8 slots; one gate/up and one down tile per worker and slot: 32 each; 32 router tiles
        assert (p["t_router"], p["t_egu"], p["t_edown"], p["k_down"]) == (32, 32, 32, 1)
    else:
        # 128 slots; 6 tiles per slot: about two per worker over the ~82 slots a uniform routing keeps busy
        assert (p["t_router"], p["t_egu"], p["t_edown"]) == (8, 6, 6) and M == 128
    h = ex["header"]
    assert h["n_empty"] / h["NT"] < (0.01 if s.batch == 1 else 0.05)   # "deep, not wide"


@pytest.mark.parametrize("over,code", [(dict(top_k=9, n_experts=8), -2), (dict(n_experts=300), -2),
                                       (dict(moe_ffn=100), -2), (dict(norm_topk=2), -1)])
def test_bad_moe_config_rejected(over, code):
    c = mpk.model_cfg(synth.SHAPES["tiny_moe"].cfg())
    for k, v in over.items():
        setattr(c, k, v)
    with pytest.raises(mpk.MpkError) as e:
        mpk.TGraph(c, 3, 16, {}, host_only=True)
    assert e.value.code == code
