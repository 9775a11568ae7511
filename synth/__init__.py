"""Seeded synthetic inputs for the decode step (shared by the oracle tests and the HIP path).

This module holds no arithmetic of the method: it only draws random numbers and
lays them out in the input formats (weights, paged KV pool, page table, token
ids, cached lengths).  Both sides receive the same tensors from here.

Recipe (one generator per tensor, so that any tensor can be re-drawn alone):

* tensor index ``i`` is drawn from ``torch.Generator().manual_seed(seed * 1_000_003 + i)``;
* indices: 0 embedding; ``1 + 11*l + j`` for layer ``l`` and
  ``j`` in (in_norm, q, k, v, q_norm, k_norm, o, post_norm, gate, up, down);
  then final_norm, lm_head, K pool, V pool, page permutation, token ids,
  cached lengths, and (mixture-of-experts shapes) the router of each layer;
  an expert shape's gate / up / down are ``[n_experts][...]`` stacks;
* matrices: fp32 ``randn * 0.02`` rounded to bf16 (round-to-nearest-even);
* RMSNorm gains: 1 (``gamma="ones"``) or ``U[0.5, 1.5]`` (``gamma="uniform"``);
* K/V: bf16 ``N(0, 1)`` at cached positions ``< L_b``; every other slot,
  including the slot the step writes and one extra page that unused
  page-table entries point at, is NaN so that a read past ``L_b`` shows;
* pages: request ``b`` owns ``ceil((L_b + 1) / P)`` pages; the pool is the
  sum of those plus the NaN page; pages are handed out in a random permutation.
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict

import torch

LAYER_TENSORS = ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o", "post_norm", "gate", "up", "down")


@dataclass(frozen=True)
class Shape:
    """A decoder shape plus the decode-step workload it is run on."""
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    qk_norm: bool
    tied_embedding: bool
    rms_eps: float
    rope_theta: float
    max_seq_len: int
    page_size: int
    batch: int
    ctx: int = 0                 # fixed cached length (when ctx_range is None)
    ctx_range: tuple | None = None   # inclusive uniform range of cached lengths
    # mixture of experts (every layer's FFN when n_experts > 0): n_experts
    # SwiGLU experts of width moe_ffn, top_k of them per token, their softmax
    # weights renormalised over the top k when norm_topk
    n_experts: int = 0
    top_k: int = 0
    moe_ffn: int = 0
    norm_topk: bool = True

    def cfg(self) -> dict:
        d = asdict(self)
        for k in ("name", "page_size", "batch", "ctx", "ctx_range"):
            d.pop(k)
        return d

    def with_(self, **kw) -> "Shape":
        d = asdict(self)
        d.update(kw)
        return Shape(**d)


# The five workloads: a tiny decoder, and Qwen3-0.6B / 8B / 32B shapes.
SHAPES = {
    "tiny": Shape("tiny", 2, 256, 4, 2, 64, 704, 1024, False, False, 1e-6, 1e4, 256, 16, 1, ctx=128),
    "qwen3_0p6b": Shape("qwen3_0p6b", 28, 1024, 16, 8, 128, 3072, 151936, True, True, 1e-6, 1e4, 1024, 64, 1,
                        ctx=512),
    "qwen3_8b": Shape("qwen3_8b", 36, 4096, 32, 8, 128, 12288, 151936, True, False, 1e-6, 1e4, 8192, 64, 1,
                      ctx=1024),
    "qwen3_8b_b16": Shape("qwen3_8b_b16", 36, 4096, 32, 8, 128, 12288, 151936, True, False, 1e-6, 1e4, 8192, 64,
                          16, ctx_range=(256, 4096)),
    "qwen3_32b": Shape("qwen3_32b", 64, 5120, 64, 8, 128, 25600, 151936, True, False, 1e-6, 1e4, 8192, 64, 1,
                       ctx=4096),
    # mixture-of-experts decoders: a tiny one, and the Qwen3-30B-A3B shape (48 layers, 128 experts of width
    # 768, 8 per token) at batch 1 and at batch 16 with ragged contexts
    "tiny_moe": Shape("tiny_moe", 2, 256, 4, 2, 64, 704, 1024, False, False, 1e-6, 1e4, 256, 16, 1, ctx=128,
                      n_experts=8, top_k=2, moe_ffn=96),
    "qwen3_30b_a3b": Shape("qwen3_30b_a3b", 48, 2048, 32, 4, 128, 6144, 151936, True, False, 1e-6, 1e4, 8192, 64, 1,
                           ctx=1024, n_experts=128, top_k=8, moe_ffn=768),
    "qwen3_30b_a3b_b16": Shape("qwen3_30b_a3b_b16", 48, 2048, 32, 4, 128, 6144, 151936, True, False, 1e-6, 1e4, 8192,
                               64, 16, ctx_range=(256, 4096), n_experts=128, top_k=8, moe_ffn=768),
}


def _gen(seed: int, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + index)
    return g


def _mat(shape, seed, index, device):
    g = _gen(seed, index, device)
    return (torch.randn(shape, generator=g, dtype=torch.float32, device=device) * 0.02).to(torch.bfloat16)


def _gain(n, seed, index, device, gamma):
    if gamma == "ones":
        return torch.ones(n, dtype=torch.bfloat16, device=device)
    g = _gen(seed, index, device)
    return (0.5 + torch.rand(n, generator=g, dtype=torch.float32, device=device)).to(torch.bfloat16)


def n_fixed(s: Shape) -> int:
    return 1 + 11 * s.n_layers


def make_weights(s: Shape, seed: int = 0, device="cpu", gamma="ones") -> dict:
    """bf16 weights, ``[out, in]`` row-major matrices, on ``device``."""
    H, d, hq, hkv, F, V = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads, s.ffn, s.vocab
    w = {"embed": _mat((V, H), seed, 0, device), "layers": []}
    shapes = {"in_norm": (H,), "q": (hq * d, H), "k": (hkv * d, H), "v": (hkv * d, H), "q_norm": (d,),
              "k_norm": (d,), "o": (H, hq * d), "post_norm": (H,), "gate": (F, H), "up": (F, H), "down": (H, F)}
    E, Fe = s.n_experts, s.moe_ffn
    if E:   # expert weights [E][...]; the router [E][H] is drawn after every other tensor (see below)
        shapes.update(gate=(E, Fe, H), up=(E, Fe, H), down=(E, H, Fe))
    for l in range(s.n_layers):
        lw = {}
        for j, name in enumerate(LAYER_TENSORS):
            idx = 1 + 11 * l + j
            if len(shapes[name]) == 1:
                lw[name] = _gain(shapes[name][0], seed, idx, device, gamma)
            else:
                lw[name] = _mat(shapes[name], seed, idx, device)
        w["layers"].append(lw)
    base = n_fixed(s)
    w["final_norm"] = _gain(H, seed, base, device, gamma)
    w["lm_head"] = None if s.tied_embedding else _mat((V, H), seed, base + 1, device)
    if E:   # router of layer l: tensor n_fixed + 7 + l, after the KV pools, page table, tokens and lengths
        for l in range(s.n_layers):
            w["layers"][l]["router"] = _mat((E, H), seed, base + 7 + l, device)
    return w


def make_seq_lens(s: Shape, seed: int = 0) -> torch.Tensor:
    if s.ctx_range is None:
        return torch.full((s.batch,), s.ctx, dtype=torch.int32)
    g = _gen(seed, n_fixed(s) + 6, "cpu")
    lo, hi = s.ctx_range
    return torch.randint(lo, hi + 1, (s.batch,), generator=g, dtype=torch.int64).to(torch.int32)


def make_token_ids(s: Shape, seed: int = 0) -> torch.Tensor:
    g = _gen(seed, n_fixed(s) + 5, "cpu")
    return torch.randint(0, s.vocab, (s.batch,), generator=g, dtype=torch.int64).to(torch.int32)


def make_kv(s: Shape, seq_lens, seed: int = 0, device="cpu") -> dict:
    """Paged K/V pools ``[n_layers, n_pages, kv_heads, P, d]`` (bf16) and the page table.

    Returns a dict with ``k_pool, v_pool, page_table [B, max_pages] int32 (CPU)``,
    ``n_pages`` (pool pages including the NaN page) and ``max_pages``.
    """
    P = s.page_size
    lens = [int(x) for x in seq_lens]
    B = len(lens)
    if any(L + 1 > s.max_seq_len for L in lens):
        raise ValueError("cached length + 1 exceeds max_seq_len")
    need = [(L + 1 + P - 1) // P for L in lens]
    n_used = sum(need)
    n_pages = n_used + 1                 # last page: NaN, target of unused entries
    max_pages = (s.max_seq_len + P - 1) // P
    g = _gen(seed, n_fixed(s) + 4, "cpu")
    perm = torch.randperm(n_used, generator=g)
    table = torch.full((B, max_pages), n_used, dtype=torch.int32)
    valid = torch.zeros(n_pages, dtype=torch.int64)   # cached tokens held by each physical page
    pos = 0
    for b in range(B):
        for j in range(need[b]):
            p = int(perm[pos]); pos += 1
            table[b, j] = p
            valid[p] = max(0, min(P, lens[b] - j * P))
    shape = (s.n_layers, n_pages, s.n_kv_heads, P, s.head_dim)
    slot = torch.arange(P).view(1, P)
    mask = (slot < valid.view(-1, 1)).view(1, n_pages, 1, P, 1).to(device)
    pools = []
    for k, idx in ((0, n_fixed(s) + 2), (1, n_fixed(s) + 3)):
        gk = _gen(seed, idx, device)
        x = torch.randn(shape, generator=gk, dtype=torch.float32, device=device)
        x = torch.where(mask, x, torch.full((), float("nan"), device=device))
        pools.append(x.to(torch.bfloat16))
        del x
    return {"k_pool": pools[0], "v_pool": pools[1], "page_table": table, "n_pages": n_pages,
            "max_pages": max_pages}


def make_inputs(s: Shape, seed: int = 0, device="cpu", gamma="ones", seq_lens=None, token_ids=None) -> dict:
    """Everything one decode step needs."""
    if seq_lens is None:
        seq_lens = make_seq_lens(s, seed)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32)
    if token_ids is None:
        token_ids = make_token_ids(s, seed)
    token_ids = torch.as_tensor(token_ids, dtype=torch.int32)
    return {"shape": s, "weights": make_weights(s, seed, device, gamma), "kv": make_kv(s, seq_lens, seed, device),
            "token_ids": token_ids, "seq_lens": seq_lens}
