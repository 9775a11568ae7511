"""Numeric oracle: one decode step of a Qwen3-shaped decoder, plain numpy on the CPU.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Shares no code with the
HIP path.

What is computed, and where the pages fix it
--------------------------------------------
MPK summary page ("MPK: A Compiler and Runtime for Mega-Kernelizing Tensor
Programs -- L2"), section 3, "Target operation, shapes & precision contract":

* MatMul tasks: bf16 inputs and outputs, fp32 accumulation.  Here the weights
  are the same bf16-rounded values the GPU reads, widened exactly; the forward
  itself runs in ``dtype`` (fp32 by default, as the plain fp32 decoder forward
  the mega-kernel is checked against; fp64 on request) with no intermediate
  bf16 rounding.
* Attention task: paged-attention decode, a ``[B, 1, H, D]`` query against a
  paged KV cache whose length varies per request.

Section 2 (Q1, the regime) and section 4 ("% peak / lower-bound derivation")
fix the workload: single-token decode of Qwen3-shaped models at batch 1-16.
Section 5 (Fig 10, techniques inventory: the fused gather-GEMM of MoE
layers) and the author's comments ("our next step is to support MoE
models") bring in mixture-of-experts layers; the plainest reading of one is
the Qwen3-MoE layer (softmax router, top-k experts, weights renormalised over
them, SwiGLU experts).
The pages name RMSNorm, RoPE and SwiGLU but do not write the decoder layer
out.  The plainest reading, the Qwen3 decoder layer, is used:

    x   = E[token]
    per layer:
      h   = RMSNorm(x; g_in)                          (eps inside the sqrt)
      q,k,v = h Wq^T, h Wk^T, h Wv^T                  (per-head reshape)
      q,k = RMSNorm per head over d (if qk_norm)      (before RoPE)
      q,k = RoPE rotate-half at position L_b          (angles in fp64)
      append k, v as position L_b; attend over L_b + 1 keys,
      kv head of q head h is floor(h / G); cached keys are already rotated
      x  += concat(o) Wo^T
      h2  = RMSNorm(x; g_post)
      x  += (silu(h2 Wg^T) * (h2 Wu^T)) Wd^T
            (mixture of experts: x += sum over the token's top-k experts e of
             w_e (silu(h2 Wg_e^T) * (h2 Wu_e^T)) Wd_e^T, w = softmax(h2 Wr^T)
             at those experts, renormalised over them -- the Qwen3-MoE layer)
    logits = RMSNorm(x; g_final) Wlm^T   (Wlm = E when tied)
    next   = argmax(logits), lowest index on ties

Paged KV layout read here: ``k_pool[layer, page, kv_head, slot, d]``; the
tokens of request ``b`` live in pages ``page_table[b, 0..n_b-1]`` with
``n_b = ceil((L_b + 1) / P)``, token ``p`` at slot ``p % P`` of page
``page_table[b, p // P]``.
"""
from __future__ import annotations

import math

import numpy as np


def widen(a, dtype=np.float32):
    """Exact widening of bf16 values to ``dtype``.

    ``a`` is either a ``uint16`` array of bf16 bit patterns (bf16 is the upper
    half of an IEEE binary32) or an already-floating array.
    """
    a = np.asarray(a)
    if a.dtype == np.uint16:
        f = (a.astype(np.uint32) << 16).view(np.float32)
        return f.astype(dtype, copy=False)
    return a.astype(dtype, copy=False)


def rms_norm(v, gamma, eps):
    """RMSNorm over the last axis: ``v / sqrt(mean(v^2) + eps) * gamma``."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * gamma


def rope_angles(pos, d, theta):
    """Rotation angles ``theta_i = pos * theta^(-2i/d)`` for ``i < d/2``, in fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = np.power(np.float64(theta), -2.0 * i / d)
    return np.float64(pos) * inv


def rope_rotate_half(v, pos, theta):
    """Rotate-half RoPE of ``v[..., d]`` at integer position ``pos``.

    Pairs are ``(i, i + d/2)``: ``u_i = v_i cos - v_{i+d/2} sin`` and
    ``u_{i+d/2} = v_{i+d/2} cos + v_i sin``.
    """
    d = v.shape[-1]
    ang = rope_angles(pos, d, theta)
    c = np.cos(ang).astype(v.dtype)
    s = np.sin(ang).astype(v.dtype)
    a, b = v[..., : d // 2], v[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(s):
    """Max-subtracted softmax over the last axis."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_one_head(q, K, Vv):
    """Single-query attention: ``softmax(K q / sqrt(d)) V`` for ``K, V: [n, d]``."""
    d = q.shape[-1]
    s = (K @ q) / np.sqrt(q.dtype.type(d))
    return softmax(s) @ Vv


def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    return silu(g) * u


def gemv(x, W):
    """``y = x W^T`` for ``W[out, in]`` (nn.Linear layout)."""
    return x @ W.T


def moe_route(logits, top_k, norm_topk):
    """Expert routing of each row of router logits ``[B, E]``.

    The probabilities are the softmax over the E experts; a token goes to the
    ``top_k`` most probable (ties to the lowest expert index), with those
    probabilities as weights, renormalised to sum to one when ``norm_topk``.
    Returns ``(ids [B, k], weights [B, k], margin [B])``: ids in decreasing
    probability, and the margin between the k-th and the (k+1)-th probability
    (how far the choice is from a tie; inf when k = E)."""
    p = softmax(logits)
    B, E = p.shape
    ids = np.zeros((B, top_k), dtype=np.int64)
    w = np.zeros((B, top_k), dtype=p.dtype)
    margin = np.full(B, np.inf)
    for b in range(B):
        order = sorted(range(E), key=lambda e: (-p[b, e], e))
        ids[b] = order[:top_k]
        w[b] = p[b, ids[b]]
        if top_k < E:
            margin[b] = float(p[b, order[top_k - 1]] - p[b, order[top_k]])
    if norm_topk:
        w = w / np.sum(w, axis=-1, keepdims=True)
    return ids, w, margin


def moe_ffn(h, router, gate, up, down, top_k, norm_topk, dtype, route_hook=None):
    """Mixture-of-experts SwiGLU FFN of rows ``h [B, H]``: router logits
    ``h router^T``, routing (``moe_route``), then for each token the sum over
    its experts e of ``w_e (silu(h gate_e^T) * (h up_e^T)) down_e^T``.
    ``gate``, ``up``, ``down`` are indexable by expert (``[E][F][H]``,
    ``[E][F][H]``, ``[E][H][F]``); only the chosen experts are read.

    ``route_hook(logits, ids, margin)``, when given, may return other expert
    ids ``[B, k]`` (or None): a near-tie between the k-th and the (k+1)-th
    probability has more than one top-k set that is correct up to rounding,
    and a caller comparing with another implementation takes that one's
    choice there.  The weights are then the softmax probabilities of the
    given experts, renormalised like ``moe_route``'s.
    Returns ``(out [B, H], logits, ids, weights, margin)``."""
    logits = gemv(h, widen(router, dtype))
    ids, w, margin = moe_route(logits, top_k, norm_topk)
    if route_hook is not None:
        forced = route_hook(logits, ids, margin)
        if forced is not None:
            ids = np.asarray(forced, dtype=np.int64)
            p = softmax(logits)
            w = np.take_along_axis(p, ids, axis=-1)
            if norm_topk:
                w = w / np.sum(w, axis=-1, keepdims=True)
    out = np.zeros_like(h)
    for b in range(h.shape[0]):
        for j in range(top_k):
            e = int(ids[b, j])
            a = swiglu(gemv(h[b], widen(gate[e], dtype)), gemv(h[b], widen(up[e], dtype)))
            out[b] += w[b, j] * gemv(a, widen(down[e], dtype))
    return out, logits, ids, w, margin


def argmax_lowest(v):
    """Index of the maximum along the last axis; ties go to the lowest index."""
    return np.argmax(v, axis=-1)


def gather_cache(pool_l, page_table_b, n_tokens, page_size, dtype):
    """Contiguous ``[kv_head, n_tokens, d]`` view of one request's cached tokens.

    ``pool_l`` is ``[n_pages, kv_head, P, d]`` for one layer.
    """
    n_pages = (n_tokens + page_size - 1) // page_size
    if n_tokens == 0:
        hk, d = pool_l.shape[1], pool_l.shape[3]
        return np.zeros((hk, 0, d), dtype=dtype)
    pages = np.asarray(page_table_b[:n_pages], dtype=np.int64)
    blk = widen(pool_l[pages], dtype)                       # [n_pages, hkv, P, d]
    blk = np.transpose(blk, (1, 0, 2, 3))                  # [hkv, n_pages, P, d]
    hk, _, P, d = blk.shape
    return blk.reshape(hk, n_pages * P, d)[:, :n_tokens, :]


def decode_step(cfg, weights, token_ids, k_pool, v_pool, page_table, seq_lens, page_size,
                dtype=np.float32, capture=None, route_hook=None):
    """One decode step of the whole batch.

    Parameters
    ----------
    cfg : mapping with ``n_layers, hidden, n_q_heads, n_kv_heads, head_dim,
        ffn, vocab, qk_norm, rms_eps, rope_theta``.
    weights : mapping with ``embed [V,H]``, ``final_norm [H]``, ``lm_head [V,H]``
        or ``None`` (tied) and ``layers``, an indexable of mappings with
        ``in_norm, q, k, v, q_norm, k_norm, o, post_norm, gate, up, down``
        (``[out, in]`` matrices).  Arrays are bf16 bit patterns (``uint16``)
        or floats; each is widened to ``dtype`` when used.
    token_ids : ``[B]`` ints.
    k_pool, v_pool : ``[n_layers, n_pages, kv_heads, P, d]`` bf16 bits / floats.
    page_table : ``[B, max_pages]`` physical page ids.
    seq_lens : ``[B]`` tokens already cached (``L_b``); the new token sits at
        position ``L_b``.
    capture : optional dict, filled with per-layer intermediates
        (``capture[l][name]``) and the new cache rows ``k_new``/``v_new``.
    route_hook : mixture of experts only, optional ``f(l, logits, ids,
        margin)`` for layer l (see ``moe_ffn``).

    Returns ``(logits [B, V], next_ids [B])``.
    """
    L = int(cfg["n_layers"]); H = int(cfg["hidden"]); hq = int(cfg["n_q_heads"])
    hkv = int(cfg["n_kv_heads"]); d = int(cfg["head_dim"])
    G = hq // hkv
    eps = dtype(cfg["rms_eps"]); theta = float(cfg["rope_theta"])
    qk_norm = bool(cfg["qk_norm"])
    token_ids = np.asarray(token_ids, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = token_ids.shape[0]

    x = widen(np.asarray(weights["embed"])[token_ids], dtype)          # [B, H]
    if capture is not None:
        capture["embed"] = x.copy()
    for l in range(L):
        Wl = weights["layers"][l]
        r = x
        h = rms_norm(r, widen(Wl["in_norm"], dtype), eps)
        q = gemv(h, widen(Wl["q"], dtype)).reshape(B, hq, d)
        k = gemv(h, widen(Wl["k"], dtype)).reshape(B, hkv, d)
        v = gemv(h, widen(Wl["v"], dtype)).reshape(B, hkv, d)
        qkv = np.concatenate([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], axis=1)
        if qk_norm:
            q = rms_norm(q, widen(Wl["q_norm"], dtype), eps)
            k = rms_norm(k, widen(Wl["k_norm"], dtype), eps)
        q = np.stack([rope_rotate_half(q[b], int(seq_lens[b]), theta) for b in range(B)])
        k = np.stack([rope_rotate_half(k[b], int(seq_lens[b]), theta) for b in range(B)])
        attn = np.zeros((B, hq, d), dtype=dtype)
        for b in range(B):
            Lb = int(seq_lens[b])
            Kc = gather_cache(k_pool[l], page_table[b], Lb, page_size, dtype)   # [hkv, Lb, d]
            Vc = gather_cache(v_pool[l], page_table[b], Lb, page_size, dtype)
            Kf = np.concatenate([Kc, k[b][:, None, :]], axis=1)                  # [hkv, Lb+1, d]
            Vf = np.concatenate([Vc, v[b][:, None, :]], axis=1)
            for hh in range(hq):
                g = hh // G
                attn[b, hh] = attention_one_head(q[b, hh], Kf[g], Vf[g])
        attn2 = attn.reshape(B, hq * d)
        o = gemv(attn2, widen(Wl["o"], dtype))
        s = r + o
        h2 = rms_norm(s, widen(Wl["post_norm"], dtype), eps)
        moe = {}
        if int(cfg.get("n_experts", 0)) > 0:
            hook = None if route_hook is None else (lambda lg, i, m, l=l: route_hook(l, lg, i, m))
            dn, rl, ids, wts, margin = moe_ffn(h2, Wl["router"], Wl["gate"], Wl["up"], Wl["down"],
                                               int(cfg["top_k"]), bool(cfg.get("norm_topk", True)), dtype,
                                               route_hook=hook)
            a = None
            moe = dict(router_logits=rl, expert_ids=ids, expert_weights=wts, route_margin=margin)
        else:
            g_ = gemv(h2, widen(Wl["gate"], dtype))
            u_ = gemv(h2, widen(Wl["up"], dtype))
            a = swiglu(g_, u_)
            dn = gemv(a, widen(Wl["down"], dtype))
        x = s + dn
        if capture is not None:
            capture[l] = dict(r=r, h=h, qkv=qkv, q=q.reshape(B, -1), k_new=k, v_new=v,
                              attn=attn2, o=o, s=s, h2=h2, a=a, d=dn, **moe)
    hf = rms_norm(x, widen(weights["final_norm"], dtype), eps)
    lm = weights["lm_head"] if weights.get("lm_head") is not None else weights["embed"]
    logits = gemv(hf, widen(lm, dtype))
    if capture is not None:
        capture["hf"] = hf
    return logits, argmax_lowest(logits)


def top2_gap(logits):
    """Per row: largest logit minus the second largest."""
    part = np.sort(logits, axis=-1)
    return part[..., -1] - part[..., -2]
