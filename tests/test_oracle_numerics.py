"""Pins for the numeric oracle (CPU only).

Each check fixes the oracle to something other than itself: closed forms,
invariants, special cases that reduce to a textbook result, independent library
routines (torch functional ops, the transformers Qwen3 / Llama decoders) and
brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import numerics as on
import synth
from tests._util import run_oracle, bf16_bits


RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    for c in (0.0, 1e-4, 0.3, -2.5, 17.0):
        v = np.full(64, c, dtype=np.float64)
        g = RNG.uniform(0.5, 1.5, 64)
        eps = 1e-6
        out = on.rms_norm(v, g, eps)
        np.testing.assert_allclose(out, c / math.sqrt(c * c + eps) * g, rtol=1e-14, atol=1e-300)


def test_rmsnorm_matches_torch_functional():
    v = RNG.standard_normal((3, 257))
    g = RNG.uniform(0.5, 1.5, 257)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (257,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(on.rms_norm(v, g, 1e-6), ref, rtol=1e-12, atol=1e-14)


def test_rmsnorm_scale_invariant():
    v = RNG.standard_normal(128)
    g = np.ones(128)
    np.testing.assert_allclose(on.rms_norm(1000.0 * v, g, 1e-6), on.rms_norm(v, g, 1e-12), rtol=1e-9)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    v = RNG.standard_normal((4, 64))
    np.testing.assert_array_equal(on.rope_rotate_half(v, 0, 1e4), v)


def test_rope_preserves_pair_norms():
    d = 128
    v = RNG.standard_normal(d)
    u = on.rope_rotate_half(v, 4097, 1e4)
    np.testing.assert_allclose(u[: d // 2] ** 2 + u[d // 2:] ** 2, v[: d // 2] ** 2 + v[d // 2:] ** 2, rtol=1e-12)


def test_rope_equals_complex_multiply():
    d, pos, theta = 64, 777, 1e4
    v = RNG.standard_normal(d)
    z = v[: d // 2] + 1j * v[d // 2:]
    ang = np.array([pos / theta ** (2 * i / d) for i in range(d // 2)])
    w = z * np.exp(1j * ang)
    u = on.rope_rotate_half(v, pos, theta)
    np.testing.assert_allclose(u, np.concatenate([w.real, w.imag]), rtol=1e-10, atol=1e-12)


def test_rope_first_pair_rotates_by_position():
    # theta^(0) = 1, so pair 0 turns by exactly `pos` radians
    v = np.zeros(32); v[0] = 1.0
    u = on.rope_rotate_half(v, 3, 1e6)
    np.testing.assert_allclose([u[0], u[16]], [math.cos(3), math.sin(3)], rtol=1e-14)


# ---------------------------------------------------------------- attention
def test_attention_single_key_returns_its_value():
    q = RNG.standard_normal(64); K = RNG.standard_normal((1, 64)); V = RNG.standard_normal((1, 64))
    np.testing.assert_allclose(on.attention_one_head(q, K, V), V[0], rtol=1e-14)


def test_attention_identical_keys_average_values():
    q = RNG.standard_normal(64); K = np.tile(RNG.standard_normal(64), (9, 1)); V = RNG.standard_normal((9, 64))
    np.testing.assert_allclose(on.attention_one_head(q, K, V), V.mean(axis=0), rtol=1e-12)


def test_attention_dominant_score_selects_value():
    d = 16
    q = np.zeros(d); q[0] = 1.0
    K = np.zeros((5, d)); K[3, 0] = 1e4
    V = RNG.standard_normal((5, d))
    np.testing.assert_allclose(on.attention_one_head(q, K, V), V[3], rtol=1e-12)


def test_attention_matches_torch_sdpa_gqa():
    hq, hkv, n, d = 8, 2, 37, 64
    q = RNG.standard_normal((hq, d)); K = RNG.standard_normal((hkv, n, d)); V = RNG.standard_normal((hkv, n, d))
    G = hq // hkv
    Kr = torch.from_numpy(np.repeat(K, G, axis=0)); Vr = torch.from_numpy(np.repeat(V, G, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], Kr, Vr)[:, 0].numpy()
    ours = np.stack([on.attention_one_head(q[h], K[h // G], V[h // G]) for h in range(hq)])
    np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- SwiGLU, argmax, widening
def test_silu_limits_and_torch():
    z = np.array([0.0, 40.0, -40.0])
    np.testing.assert_allclose(on.silu(z), [0.0, 40.0, 0.0], atol=1e-15)
    z = RNG.standard_normal(100) * 5
    np.testing.assert_allclose(on.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-12)
    g = RNG.standard_normal(10); u = RNG.standard_normal(10)
    np.testing.assert_allclose(on.swiglu(g, u), g / (1 + np.exp(-g)) * u, rtol=1e-15)


def test_argmax_ties_go_to_lowest_index():
    v = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]])
    assert list(on.argmax_lowest(v)) == [1, 0]


def test_widen_bf16_bits_exact():
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    np.testing.assert_array_equal(on.widen(bf16_bits(x)), x.float().numpy())


def test_gemv_brute_force():
    x = RNG.standard_normal((2, 7)); W = RNG.standard_normal((5, 7))
    ref = np.array([[sum(x[b, k] * W[n, k] for k in range(7)) for n in range(5)] for b in range(2)])
    np.testing.assert_allclose(on.gemv(x, W), ref, rtol=1e-13)


def test_gather_cache_brute_force():
    P, hkv, d, n_pages = 4, 2, 3, 6
    pool = RNG.standard_normal((n_pages, hkv, P, d))
    table = np.array([5, 2, 0, 3])
    for n in (0, 1, 4, 5, 11):
        got = on.gather_cache(pool, table, n, P, np.float64)
        assert got.shape == (hkv, n, d)
        for g in range(hkv):
            for p in range(n):
                np.testing.assert_array_equal(got[g, p], pool[table[p // P], g, p % P])


# ---------------------------------------------------------------- whole decode step vs transformers
def _hf_model(s, w, arch):
    from transformers import Qwen3Config, Qwen3ForCausalLM, LlamaConfig, LlamaForCausalLM
    common = dict(vocab_size=s.vocab, hidden_size=s.hidden, intermediate_size=s.ffn, num_hidden_layers=s.n_layers,
                  num_attention_heads=s.n_q_heads, num_key_value_heads=s.n_kv_heads, head_dim=s.head_dim,
                  rms_norm_eps=s.rms_eps, max_position_embeddings=s.max_seq_len,
                  rope_parameters={"rope_type": "default", "rope_theta": s.rope_theta},
                  tie_word_embeddings=s.tied_embedding, attention_bias=False)
    if arch == "qwen3":
        m = Qwen3ForCausalLM(Qwen3Config(**common, attn_implementation="eager"))
    elif arch == "qwen3_moe":
        from transformers import Qwen3MoeConfig, Qwen3MoeForCausalLM
        cfg = Qwen3MoeConfig(**common, num_experts=s.n_experts, num_experts_per_tok=s.top_k,
                             moe_intermediate_size=s.moe_ffn, norm_topk_prob=s.norm_topk, decoder_sparse_step=1,
                             mlp_only_layers=[], attn_implementation="eager")
        cfg._experts_implementation = "eager"   # the per-expert loop (the grouped-GEMM path has no fp64)
        m = Qwen3MoeForCausalLM(cfg)
    else:
        m = LlamaForCausalLM(LlamaConfig(**common, mlp_bias=False, attn_implementation="eager"))
    m = m.double().eval()
    # The stock rotary module evaluates its angles in fp32; give it fp64 angles
    # (same inverse-frequency formula and cos/sin layout).
    inv = 1.0 / (s.rope_theta ** (torch.arange(0, s.head_dim, 2, dtype=torch.float64) / s.head_dim))

    def rotary64(x, position_ids):
        fr = position_ids[:, :, None].double() * inv[None, None, :]
        emb = torch.cat((fr, fr), dim=-1)
        return emb.cos().to(x.dtype), emb.sin().to(x.dtype)
    m.model.rotary_emb.forward = rotary64
    f = lambda t: t.double()
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(f(w["embed"]))
        for l, lw in enumerate(w["layers"]):
            L = m.model.layers[l]
            L.input_layernorm.weight.copy_(f(lw["in_norm"]))
            L.self_attn.q_proj.weight.copy_(f(lw["q"])); L.self_attn.k_proj.weight.copy_(f(lw["k"]))
            L.self_attn.v_proj.weight.copy_(f(lw["v"])); L.self_attn.o_proj.weight.copy_(f(lw["o"]))
            if arch in ("qwen3", "qwen3_moe"):
                L.self_attn.q_norm.weight.copy_(f(lw["q_norm"])); L.self_attn.k_norm.weight.copy_(f(lw["k_norm"]))
            L.post_attention_layernorm.weight.copy_(f(lw["post_norm"]))
            if arch == "qwen3_moe":   # router [E][H]; experts: gate and up stacked [E][2F][H], down [E][H][F]
                L.mlp.gate.weight.copy_(f(lw["router"]))
                L.mlp.experts.gate_up_proj.copy_(torch.cat([f(lw["gate"]), f(lw["up"])], dim=1))
                L.mlp.experts.down_proj.copy_(f(lw["down"]))
            else:
                L.mlp.gate_proj.weight.copy_(f(lw["gate"])); L.mlp.up_proj.weight.copy_(f(lw["up"]))
                L.mlp.down_proj.weight.copy_(f(lw["down"]))
        m.model.norm.weight.copy_(f(w["final_norm"]))
        if not s.tied_embedding:
            m.lm_head.weight.copy_(f(w["lm_head"]))
    return m


def _hf_logits(s, inp, m):
    from transformers import DynamicCache
    kv = inp["kv"]; P = s.page_size
    rows = []
    for b in range(s.batch):
        Lb = int(inp["seq_lens"][b])
        cache = DynamicCache()
        for l in range(s.n_layers):
            Ks = on.gather_cache(bf16_bits(kv["k_pool"][l]), kv["page_table"][b].numpy(), Lb, P, np.float64)
            Vs = on.gather_cache(bf16_bits(kv["v_pool"][l]), kv["page_table"][b].numpy(), Lb, P, np.float64)
            cache.update(torch.from_numpy(Ks)[None], torch.from_numpy(Vs)[None], l)
        ids = inp["token_ids"][b:b + 1].long()[None]
        with torch.no_grad():
            out = m(input_ids=ids, position_ids=torch.tensor([[Lb]]), past_key_values=cache, use_cache=True)
        rows.append(out.logits[0, -1].numpy())
    return np.stack(rows)


SMALL_QK = synth.Shape("small_qk", 2, 128, 4, 2, 32, 192, 300, True, False, 1e-6, 1e4, 128, 16, 3,
                       ctx_range=(0, 70))


@pytest.mark.parametrize("shape,arch,gamma", [
    (SMALL_QK, "qwen3", "uniform"),
    (SMALL_QK.with_(tied_embedding=True, rope_theta=1e6), "qwen3", "uniform"),
    (synth.SHAPES["tiny"].with_(batch=2, ctx_range=(5, 140), ctx=0), "llama", "uniform"),
    (SMALL_QK.with_(n_experts=6, top_k=2, moe_ffn=48), "qwen3_moe", "uniform"),
    (SMALL_QK.with_(n_experts=5, top_k=3, moe_ffn=40, norm_topk=False, batch=2), "qwen3_moe", "ones"),
])
def test_decode_step_matches_transformers(shape, arch, gamma):
    inp = synth.make_inputs(shape, seed=3, gamma=gamma)
    logits, nxt = run_oracle(inp, dtype=np.float64)
    m = _hf_model(shape, inp["weights"], arch)
    ref = _hf_logits(shape, inp, m)
    # The library evaluates RMSNorm and the softmax in fp32 even in an fp64
    # model, so agreement is at fp32 level (~1e-7 absolute on logits of ~0.3);
    # the planted-error cases the other pins target are orders larger.
    np.testing.assert_allclose(logits, ref, rtol=1e-5, atol=2e-6)
    np.testing.assert_array_equal(nxt, ref.argmax(-1))


def test_fp32_oracle_close_to_fp64():
    s = synth.SHAPES["tiny"].with_(batch=3, ctx_range=(0, 200), ctx=0)
    inp = synth.make_inputs(s, seed=11, gamma="uniform")
    l32, _ = run_oracle(inp, dtype=np.float32)
    l64, _ = run_oracle(inp, dtype=np.float64)
    assert np.all(np.isfinite(l32))
    np.testing.assert_allclose(l32, l64, rtol=1e-4, atol=1e-4)


def test_oracle_never_reads_poisoned_slots():
    # every slot at or past L_b is NaN; a finite result shows none was read
    s = synth.SHAPES["tiny"].with_(batch=4, ctx_range=(0, 60), ctx=0)
    inp = synth.make_inputs(s, seed=5)
    assert torch.isnan(inp["kv"]["k_pool"].float()).any()
    logits, _ = run_oracle(inp)
    assert np.all(np.isfinite(logits))


# ---------------------------------------------------------------- mixture of experts
def test_moe_route_hand_values():
    # probabilities 0.1, 0.2, 0.3, 0.4 (logits ln 1 .. ln 4): the top 2 are experts 3 and 2
    lg = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    ids, w, margin = on.moe_route(lg, 2, True)
    assert ids.tolist() == [[3, 2]]
    np.testing.assert_allclose(w, [[0.4 / 0.7, 0.3 / 0.7]], rtol=1e-12)
    np.testing.assert_allclose(margin, [0.1], rtol=1e-12)
    ids, w, _ = on.moe_route(lg, 2, False)
    np.testing.assert_allclose(w, [[0.4, 0.3]], rtol=1e-12)
    # a tie at the cut goes to the lower expert index; top-k = E has no margin
    ids, w, margin = on.moe_route(np.array([[0.0, 1.0, 1.0, 0.0]]), 1, True)
    assert ids.tolist() == [[1]] and margin[0] == 0.0 and w[0, 0] == 1.0
    _, _, margin = on.moe_route(lg, 4, True)
    assert margin[0] == np.inf


def test_single_expert_moe_is_the_dense_ffn():
    # one expert chosen with weight 1: exactly the SwiGLU FFN of that expert
    H, F = 16, 24
    h = RNG.standard_normal((3, H))
    g, u, dn = (RNG.standard_normal(sh) * 0.2 for sh in ((1, F, H), (1, F, H), (1, H, F)))
    out, _, ids, w, _ = on.moe_ffn(h, RNG.standard_normal((1, H)), g, u, dn, 1, True, np.float64)
    dense = np.stack([on.gemv(on.swiglu(on.gemv(x, g[0]), on.gemv(x, u[0])), dn[0]) for x in h])
    assert np.all(ids == 0) and np.all(w == 1.0)
    np.testing.assert_array_equal(out, dense)


def test_moe_reads_only_the_chosen_experts():
    # experts outside each token's top k are NaN: a finite result shows none was used
    H, F, E = 8, 12, 6
    h = RNG.standard_normal((2, H))
    router = RNG.standard_normal((E, H))
    ids, _, _ = on.moe_route(on.gemv(h, router), 2, True)
    g, u, dn = (np.full(sh, np.nan) for sh in ((E, F, H), (E, F, H), (E, H, F)))
    for e in set(ids.ravel().tolist()):
        g[e], u[e], dn[e] = (RNG.standard_normal(x.shape[1:]) for x in (g, u, dn))
    out, *_ = on.moe_ffn(h, router, g, u, dn, 2, True, np.float64)
    assert np.all(np.isfinite(out))
