// Host-side tGraph builder (see builder.h for the method and its sources).
#include "builder.h"

#include <algorithm>
#include <cmath>
#include <array>
#include <deque>
#include <map>

namespace mpk {

namespace {

Box box(int32_t tensor, std::initializer_list<int32_t> lo, std::initializer_list<int32_t> hi) {
  Box b;
  b.tensor = tensor;
  for (int i = 0; i < 4; ++i) { b.lo[i] = 0; b.hi[i] = 1; }
  int i = 0;
  for (int32_t v : lo) b.lo[i++] = v;
  i = 0;
  for (int32_t v : hi) b.hi[i++] = v;
  return b;
}

bool overlaps(const Box& a, const Box& b) {
  if (a.tensor != b.tensor) return false;
  for (int i = 0; i < 4; ++i)
    if (!(a.lo[i] < b.hi[i] && b.lo[i] < a.hi[i])) return false;
  return true;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Kernel-side capacities (LDS budget of one workgroup).
constexpr int64_t kMaxTileAcc = 8192;     // fp32 accumulators of one projection tile
constexpr int64_t kMaxStagedK = 26624;    // batch-1 activation vector staged in LDS
constexpr int64_t kMaxSplitPages = 4096;  // page ids staged per attention split

}  // namespace

int resolve_params(const mpk_model_cfg& c, int32_t B, int32_t P, const mpk_build_params* in, int32_t n_cus,
                   Params* out, std::string* err) {
  auto bad = [&](const char* m) { *err = m; return (int)MPK_ERR_INVALID_ARG; };
  auto uns = [&](const char* m) { *err = m; return (int)MPK_ERR_UNSUPPORTED; };
  if (c.n_layers < 1 || c.hidden < 8 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.ffn < 8 || c.vocab < 1 ||
      c.max_seq_len < 1)
    return bad("model config: sizes must be positive");
  if (c.n_q_heads % c.n_kv_heads) return bad("model config: n_q_heads must be a multiple of n_kv_heads");
  if (c.head_dim != 64 && c.head_dim != 128) return uns("head_dim must be 64 or 128");
  if (c.hidden % 8 || c.ffn % 8) return uns("hidden and ffn must be multiples of 8");
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f)) return bad("rms_eps and rope_theta must be positive");
  if (c.qk_norm != 0 && c.qk_norm != 1) return bad("qk_norm must be 0 or 1");
  if (c.tied_embedding != 0 && c.tied_embedding != 1) return bad("tied_embedding must be 0 or 1");
  if (c.n_q_heads / c.n_kv_heads > 16) return uns("more than 16 query heads per kv head");
  if (B < 1 || B > 16) return uns("batch must be in 1..16");
  // the matrix-core tiles (batch > 1) walk the contraction in whole 32-element
  // steps, and a k-split range starts on a 32-element (128-byte) boundary of
  // the fp32 activation rows, so both inputs of a projection must be whole
  // steps (the attention output, hq x d, always is)
  if (B > 1 && (c.hidden % 32 || c.ffn % 32)) return uns("at batch > 1, hidden and ffn must be multiples of 32");
  if (P != 16 && P != 32 && P != 64) return uns("page_size must be 16, 32 or 64");
  if (c.n_experts < 0 || c.n_experts > 256) return uns("n_experts must be in 0..256");
  if (c.n_experts > 0) {
    if (c.top_k < 1 || c.top_k > 16 || c.top_k > c.n_experts) return uns("top_k must be in 1..min(16, n_experts)");
    if (c.moe_ffn < 8 || c.moe_ffn % 8 || (B > 1 && c.moe_ffn % 32))
      return uns("moe_ffn must be a positive multiple of 8 (of 32 at batch > 1)");
    if (c.norm_topk != 0 && c.norm_topk != 1) return bad("norm_topk must be 0 or 1");
  }
  mpk_build_params z = {};
  const mpk_build_params& p = in ? *in : z;
  if (p.fusion_order < 0 || p.fusion_order > 1) return uns("fusion_order must be 0 (Def 4.1 then Def 4.2) or 1 (none)");
  if (p.aot_policy != 0) return uns("only AOT policy 0 (round-robin in linear order) is implemented");
  if (p.attn_jit < 0 || p.attn_jit > 3) return bad("attn_jit must be 0, 1, 2 or 3");
  if (p.weight_preload < 0 || p.weight_preload > 3) return bad("weight_preload must be 0, 1, 2 or 3");
  Params r;
  // scheduling policy: 1 is the hybrid policy (attention JIT, the rest
  // AOT), 3 every task JIT, 2 every task AOT.  The default is AOT at every
  // batch: an attention task sizes its split from the lengths at run time,
  // so static placement is already balanced, and it measured faster than
  // the hybrid policy at the 8B shape, batch 16 (7.41 against 7.76 ms)
  r.jit_all = p.attn_jit == 3;
  r.jit_attn = r.jit_all || p.attn_jit == 1;
  r.preload = p.weight_preload != 2;
  r.lookahead = p.weight_preload == 3;
  if (p.coarse_events < 0 || p.coarse_events > 1) return bad("coarse_events must be 0 or 1");
  r.coarse = p.coarse_events == 1;
  r.fusion = p.fusion_order;
  if (p.attn_split_pages < 0) return bad("attn_split_pages must not be negative");
  r.split_pages = p.attn_split_pages > 0 ? p.attn_split_pages : 1;
  // default scheduler count: none when nothing is JIT (every compute unit
  // is a worker), else the largest S <= 16 that divides the worker count, so
  // that every scheduler deals over the same number of workers
  auto workers_for = [&](int32_t S) { return p.n_workers > 0 ? p.n_workers : n_cus - (S + 3) / 4; };
  if (p.n_sched_waves > 0) {
    r.S_sched = p.n_sched_waves;
  } else if (!r.jit_attn) {
    r.S_sched = 0;
  } else {
    r.S_sched = 1;
    for (int32_t S = 16; S >= 1; --S)
      if (workers_for(S) > 0 && workers_for(S) % S == 0) { r.S_sched = S; break; }
  }
  r.W = workers_for(r.S_sched);
  if (r.W < 1) return bad("no worker workgroups left");
  r.q = p.quantum > 0 ? p.quantum : (B == 1 ? 1 : 16);
  const int64_t G = c.n_q_heads / c.n_kv_heads, d = c.head_dim, Sg = (G + 2) * d;
  const int64_t H = c.hidden, F = c.ffn, V = c.vocab, hkv = c.n_kv_heads;
  // k-splits: at batch > 1 a tile's activation slice costs 4 B per k and
  // request (fp32), as much as 16 rows of bf16 weights; splitting k shrinks
  // it while the column tiles grow to keep one tile per worker (defaults:
  // the fastest of a sweep at the 8B shape, batch 16; the q/k/v projection's
  // narrow column tiles gain nothing from it; a tile count given without its
  // k-split keeps the default only if it divides)
  r.K_qkv = p.k_qkv > 0 ? p.k_qkv : 1;
  // (the O projection's k-ranges follow the kv groups: with K_o dividing
  // n_kv_heads an attention task feeds one range, so its tiles trigger one
  // event and the graph stays narrow -- K_o = 3 over 8 groups gave 13% empty
  // tasks at the 8B shape, batch 16, against 5% with 4)
  int32_t ko_def = 1;
  for (int32_t k = 4; k >= 2; --k)
    if (c.n_kv_heads % k == 0 && (p.t_o <= 0 || p.t_o % k == 0)) { ko_def = k; break; }
  r.K_o = p.k_o > 0 ? p.k_o : (B > 1 ? ko_def : 1);
  r.K_down = p.k_down > 0 ? p.k_down : (B > 1 && c.n_experts == 0 && (p.t_down <= 0 || p.t_down % 3 == 0) ? 3 : 1);
  // (a batch > 1 norm task stages the gain, the residual row and every plane
  // of its input in LDS: the default splits shrink, the larger first, until
  // that takes at most 128 KB, leaving the rest of the 160 KB to the
  // accumulators, page ids and control words; splits given stay as given)
  if (B > 1) {
    auto kb = [](int64_t bytes) { return (bytes + 1023) / 1024 * 1024; };
    auto fits = [&]() { return kb(H * 2) + (1 + std::max(r.K_o, r.K_down)) * kb(H * 4) <= 128 * 1024; };
    while (!fits()) {
      const bool can_o = p.k_o <= 0 && r.K_o > 1, can_d = p.k_down <= 0 && r.K_down > 1;
      if (can_o && (r.K_o >= r.K_down || !can_d)) {
        int32_t k = r.K_o - 1;
        while (k > 1 && (c.n_kv_heads % k || (p.t_o > 0 && p.t_o % k))) --k;
        r.K_o = k;
      } else if (can_d) {
        int32_t k = r.K_down - 1;
        while (k > 1 && p.t_down > 0 && p.t_down % k) --k;
        r.K_down = k;
      } else {
        break;   // (the layout check refuses the shape)
      }
    }
  }
  if (c.n_experts > 0 && r.K_down != 1)
    return uns("k_down must be 1 with experts (their outputs accumulate into one plane)");
  if (B == 1 && (r.K_qkv != 1 || r.K_o != 1 || r.K_down != 1))
    return uns("k-splits need batch > 1 (a batch-1 tile stages its whole input)");
  if (r.K_qkv > cdiv(H, 32) || r.K_o > cdiv((int64_t)c.n_q_heads * d, 32) || r.K_down > cdiv(F, 32))
    return bad("a k-split finer than 32 elements");
  if (p.t_qkv > 0) {
    if (p.t_qkv % (hkv * r.K_qkv)) return bad("t_qkv must be a multiple of n_kv_heads x k_qkv");
    r.T_qkv = p.t_qkv;
  } else {
    int64_t tpg = std::max<int64_t>(1, std::min<int64_t>(r.W / (hkv * r.K_qkv), cdiv(Sg, r.q)));
    r.T_qkv = (int32_t)(tpg * hkv * r.K_qkv);
  }
  // default: one tile per worker (W / K column tiles x K k-ranges), more
  // column tiles (in steps of W / K) while a tile's accumulators (columns x
  // rows per column x batch) exceed the LDS budget
  auto dflt = [&](int32_t v, int64_t N, int64_t rpc, int64_t K) {
    if (v > 0) return v % K ? -1 : v;
    const int64_t U = cdiv(N, r.q), Wk = std::max<int64_t>(1, r.W / K);
    int64_t T = std::min<int64_t>(Wk, U);
    while (T < U && r.q * cdiv(U, T) * rpc * B > kMaxTileAcc) T = std::min<int64_t>(U, T + Wk);
    return (int32_t)(T * K);
  };
  r.T_o = dflt(p.t_o, H, 1, r.K_o);
  r.T_gu = dflt(p.t_gu, F, 2, 1);
  r.T_down = dflt(p.t_down, H, 1, r.K_down);
  r.T_lm = dflt(p.t_lm, V, 1, 1);
  if (r.T_o < 0 || r.T_down < 0) return bad("t_o / t_down must be multiples of k_o / k_down");
  if (c.n_experts > 0) {
    // mixture of experts: router tiles on the column quantum (about W / 8);
    // per expert slot, gate/up and down tiles so that the slots' tiles make
    // one task per worker at batch 1 (every slot is busy: W / slots each) and
    // about two at batch > 1 over the slots that are busy when the batch
    // routes uniformly, E (1 - (1 - k/E)^B) of them -- an idle slot's tiles
    // finish at once, and two rounds leave a short tail (30B-A3B shape,
    // batch 16: 82 busy slots of 128, 6 tiles each); more tiles while a tile's
    // accumulators (columns x rows per column x batch) exceed the budget
    const int64_t E = c.n_experts, Fe = c.moe_ffn, M = moe_slots(c, B);
    const double busy = (double)E * (1.0 - std::pow(1.0 - (double)c.top_k / (double)E, (double)B));
    auto per_slot = [&](int32_t v, int64_t N, int64_t rpc) {
      if (v > 0) return (int64_t)v;
      const int64_t U = cdiv(N, r.q);
      const int64_t step = B == 1 ? std::max<int64_t>(1, r.W / M)
                                  : std::max<int64_t>(1, (int64_t)(2.0 * r.W / std::max(1.0, busy)));
      int64_t T = std::min<int64_t>(step, U);
      while (T < U && r.q * cdiv(U, T) * rpc * B > kMaxTileAcc) T = std::min<int64_t>(U, T + 1);
      return T;
    };
    const int64_t Tr = p.t_router > 0 ? p.t_router : std::min<int64_t>(cdiv(E, r.q), std::max<int64_t>(1, r.W / 8));
    const int64_t Tg = per_slot(p.t_egu, Fe, 2), Td = per_slot(p.t_edown, H, 1);
    struct { int64_t T, N, rpc; const char* name; } moe_ops[] = {
        {Tr, E, 1, "t_router"}, {Tg, Fe, 2, "t_egu"}, {Td, H, 1, "t_edown"}};
    for (auto& o : moe_ops) {
      if (o.T < 1 || o.T > cdiv(o.N, r.q)) { *err = std::string(o.name) + ": tile count out of range"; return MPK_ERR_INVALID_ARG; }
      if (r.q * cdiv(cdiv(o.N, r.q), o.T) * o.rpc * B > kMaxTileAcc) {
        *err = std::string(o.name) + ": tile too wide (columns x rows x batch must stay within 8192 accumulators)";
        return MPK_ERR_UNSUPPORTED;
      }
    }
    if (M * std::max(Tg, Td) > 65535) return uns("more than 65535 expert tiles per layer");
    r.T_router = (int32_t)Tr; r.T_egu = (int32_t)Tg; r.T_edown = (int32_t)Td;
  }
  int64_t max_pages = cdiv(c.max_seq_len, P);
  // S_attn = M, the attention slots of a kv group (dealt to the requests by
  // page count when the step runs); at batch 1 they are the splits
  if (p.s_attn > 0) {
    r.S_attn = p.s_attn;
    if (r.S_attn < B) return bad("s_attn: fewer attention slots per kv group than requests");
  } else if (B > 1) {
    // one attention task per worker, at most one slot per page of each request
    r.S_attn = (int32_t)std::max<int64_t>(B, std::min<int64_t>(r.W / hkv, (int64_t)B * max_pages));
  } else {
    // one attention task per worker, as at batch > 1: the request's split
    // count is decided when the step runs (at most one split per page,
    // attn_split_pages pages at least, and no more than the split combine can
    // stage), and with W attention tasks every worker runs one task of each
    // operator of a layer (8B shape: 4.06 against 4.19 ms with 8 slots)
    r.S_attn = (int32_t)std::max<int64_t>(1, std::min<int64_t>(r.W / hkv, max_pages));
  }
  if (r.T_qkv / (hkv * r.K_qkv) > cdiv(Sg, r.q)) return bad("t_qkv: more tiles per kv group than column quanta");
  // (column tiles per operator)
  struct { int64_t T, N, rows_per_col; const char* name; } ops[] = {
      {r.T_qkv / (hkv * r.K_qkv), Sg, 1, "t_qkv"}, {r.T_o / r.K_o, H, 1, "t_o"}, {r.T_gu, F, 2, "t_gu"},
      {r.T_down / r.K_down, H, 1, "t_down"}, {r.T_lm, V, 1, "t_lm"}};
  for (auto& o : ops) {
    if (o.T < 1 || o.T > cdiv(o.N, r.q)) { *err = std::string(o.name) + ": tile count out of range"; return MPK_ERR_INVALID_ARG; }
    if (o.T > 65535) { *err = std::string(o.name) + ": more than 65535 tiles"; return MPK_ERR_INVALID_ARG; }
    int64_t widest = r.q * cdiv(cdiv(o.N, r.q), o.T);
    if (widest * o.rows_per_col * B > kMaxTileAcc) {
      *err = std::string(o.name) + ": tile too wide (columns x rows x batch must stay within 8192 accumulators)";
      return MPK_ERR_UNSUPPORTED;
    }
  }
  if (r.S_attn < 1 || r.S_attn > 65535) return bad("s_attn out of range");
  if (max_pages > kMaxSplitPages) return uns("max_seq_len / page_size above 4096 pages");
  if (B == 1 && std::max<int64_t>(std::max<int64_t>(H, F), (int64_t)c.n_q_heads * d) > kMaxStagedK)
    return uns("a projection input longer than 26624 elements");
  *out = r;
  return MPK_OK;
}

void decompose(const mpk_model_cfg& c, int32_t B, const Params& p, std::vector<TaskDef>* tasks_out) {
  std::vector<TaskDef>& tasks = *tasks_out;
  tasks.clear();
  const int32_t L = c.n_layers, H = c.hidden, hq = c.n_q_heads, hkv = c.n_kv_heads, d = c.head_dim;
  const int32_t F = c.ffn, V = c.vocab, S = p.S_attn, G = hq / hkv, Sg = (G + 2) * d, maxs = c.max_seq_len;
  const bool fused = fused_norm(B);
  auto add = [&](int32_t type, int32_t layer, int32_t c0, int32_t c1, int32_t c2, std::vector<Box> ins,
                 std::vector<Box> outs) {
    TaskDef t;
    t.type = type; t.layer = layer; t.c[0] = c0; t.c[1] = c1; t.c[2] = c2;
    t.ins = std::move(ins); t.outs = std::move(outs);
    tasks.push_back(std::move(t));
  };
  auto full = [&](int32_t tensor, int32_t n) { return box(tensor, {0, 0}, {B, n}); };
  // batch > 1: one embedding / norm task per request b (coords (b,), output
  // row b); norm tasks declare all B rows of their inputs so that the B tasks
  // of an operator share one event
  auto row = [&](int32_t tensor, int32_t b, int32_t n) { return box(tensor, {b, 0}, {b + 1, n}); };
  // q/k/v, O and down outputs: one plane of partial sums per k-range,
  // [plane][b][column]; their readers take all planes
  auto planes = [&](int32_t tensor, int32_t k, int32_t n) { return box(tensor, {0, 0, 0}, {k, B, n}); };
  const int32_t Kq = p.K_qkv, Ko = p.K_o, Kd = p.K_down;
  const int32_t E = c.n_experts, Fe = c.moe_ffn, M = moe_slots(c, B), rec = route_words(B);
  const bool moe = E > 0;
  // The mixture-of-experts FFN of layer l: ROUTER tiles (logits; at batch 1
  // also the residual add + RMSNorm, tile 0 storing s_l and h2_l), then per
  // expert slot s EXPERT_GU tiles (tile 0 writes the slot's route record)
  // and EXPERT_DOWN tiles, which add into d_l and read only their slot's
  // record and gate/up output.  d_l starts the step at zero: the task that
  // stores s_l (router tile 0 at batch 1, MLP_NORM b at batch > 1, row b)
  // zeroes it; d_l and s_l have the same readers, so this adds no event.
  auto moe_layer = [&](int32_t l, const std::vector<Box>& mid) {
    auto t = [&](int32_t k) { return layer_tensor(l, k); };
    for (int32_t n = 0; n < p.T_router; ++n) {
      int32_t elo, ehi;
      tile_range(E, p.q, p.T_router, n, &elo, &ehi);
      std::vector<Box> outs = {box(t(L_RLOG), {0, elo}, {B, ehi})};
      if (fused && n == 0) {
        outs.push_back(full(t(L_S), H));
        outs.push_back(full(t(L_H2), H));
        outs.push_back(planes(t(L_D), 1, H));
      }
      add(MPK_TASK_ROUTER, l, n, 0, 0, fused ? mid : std::vector<Box>{full(t(L_H2), H)}, outs);
    }
    for (int32_t s = 0; s < M; ++s)
      for (int32_t n = 0; n < p.T_egu; ++n) {
        int32_t lo, hi;
        tile_range(Fe, p.q, p.T_egu, n, &lo, &hi);
        std::vector<Box> outs = {box(t(L_A), {s, 0, lo}, {s + 1, B, hi})};
        if (n == 0) outs.push_back(box(t(L_ROUTE), {s, 0}, {s + 1, rec}));
        add(MPK_TASK_EXPERT_GU, l, s, n, 0, {full(t(L_RLOG), E), full(t(L_H2), H)}, outs);
      }
    for (int32_t s = 0; s < M; ++s)
      for (int32_t n = 0; n < p.T_edown; ++n) {
        int32_t lo, hi;
        tile_range(H, p.q, p.T_edown, n, &lo, &hi);
        add(MPK_TASK_EXPERT_DOWN, l, s, n, 0, {box(t(L_ROUTE), {s, 0}, {s + 1, rec}), box(t(L_A), {s, 0, 0}, {s + 1, B, Fe})},
            {box(t(L_D), {0, 0, lo}, {1, B, hi})});
      }
  };
  if (!fused)
    for (int32_t b = 0; b < B; ++b) add(MPK_TASK_EMBED, -1, b, 0, 0, {}, {row(T_E, b, H)});
  for (int32_t l = 0; l < L; ++l) {
    auto t = [&](int32_t k) { return layer_tensor(l, k); };
    std::vector<Box> prev;
    if (l > 0) prev = {full(layer_tensor(l - 1, L_S), H), planes(layer_tensor(l - 1, L_D), Kd, H)};
    if (!fused)
      for (int32_t b = 0; b < B; ++b)
        add(MPK_TASK_ATTN_NORM, l, b, 0, 0, l ? prev : std::vector<Box>{full(T_E, H)},
            {row(t(L_R), b, H), row(t(L_H), b, H)});
    // tile n: kv group n / tpg, column tile (n mod tpg) / Kq, k-range n mod Kq
    const int32_t tpg = p.T_qkv / hkv;
    for (int32_t n = 0; n < p.T_qkv; ++n) {
      const int32_t g = n / tpg, j = (n % tpg) / Kq, ks = n % Kq;
      int32_t lo, hi, klo, khi;
      tile_range(Sg, p.q, tpg / Kq, j, &lo, &hi);
      tile_range(H, 32, Kq, ks, &klo, &khi);
      std::vector<Box> outs = {box(t(L_QKV), {ks, 0, g * Sg + lo}, {ks + 1, B, g * Sg + hi})};
      if (fused && n == 0) outs.push_back(full(t(L_R), H));
      // (coarse: the operator-level graph, where a task waits for the whole
      // previous operator, so a k-split tile declares its whole input row)
      add(MPK_TASK_QKV, l, n, 0, 0,
          fused ? prev : std::vector<Box>{p.coarse ? full(t(L_H), H) : box(t(L_H), {0, klo}, {B, khi})}, outs);
    }
    // attention task (j, g) is slot j of kv group g; the request a slot
    // serves is decided at run time from the sequence lengths, so every task
    // declares its whole group (all B rows)
    for (int32_t g = 0; g < hkv; ++g)
      for (int32_t s = 0; s < S; ++s) {
        std::vector<Box> outs = {box(t(L_PART), {0, g, 0, 0}, {1, g + 1, S, G * (d + 2)}),
                                 box(t(L_ATTN), {0, g * G * d}, {B, (g + 1) * G * d}),
                                 box(t(L_KC), {0, 0, g, 0}, {B, maxs, g + 1, d}),
                                 box(t(L_VC), {0, 0, g, 0}, {B, maxs, g + 1, d})};
        add(MPK_TASK_ATTN, l, s, g, 0,
            {p.coarse ? box(t(L_QKV), {0, 0, 0}, {Kq, B, hkv * Sg})
                      : box(t(L_QKV), {0, 0, g * Sg}, {Kq, B, (g + 1) * Sg})},
            outs);
      }
    for (int32_t n = 0; n < p.T_o; ++n) {   // column tile n / Ko, k-range n mod Ko
      int32_t lo, hi, klo, khi;
      tile_range(H, p.q, p.T_o / Ko, n / Ko, &lo, &hi);
      tile_range(hq * d, 32, Ko, n % Ko, &klo, &khi);
      add(MPK_TASK_OPROJ, l, n, 0, 0, {p.coarse ? full(t(L_ATTN), hq * d) : box(t(L_ATTN), {0, klo}, {B, khi})},
          {box(t(L_O), {n % Ko, 0, lo}, {n % Ko + 1, B, hi})});
    }
    const std::vector<Box> mid = {full(t(L_R), H), planes(t(L_O), Ko, H)};
    if (!fused)
      for (int32_t b = 0; b < B; ++b) {
        std::vector<Box> outs = {row(t(L_S), b, H), row(t(L_H2), b, H)};
        if (moe) outs.push_back(box(t(L_D), {0, b, 0}, {1, b + 1, H}));
        add(MPK_TASK_MLP_NORM, l, b, 0, 0, mid, outs);
      }
    if (moe) {
      moe_layer(l, mid);
      continue;
    }
    for (int32_t n = 0; n < p.T_gu; ++n) {
      int32_t lo, hi;
      tile_range(F, p.q, p.T_gu, n, &lo, &hi);
      std::vector<Box> outs = {box(t(L_A), {0, lo}, {B, hi})};
      if (fused && n == 0) outs.push_back(full(t(L_S), H));
      add(MPK_TASK_GATEUP, l, n, 0, 0, fused ? mid : std::vector<Box>{full(t(L_H2), H)}, outs);
    }
    for (int32_t n = 0; n < p.T_down; ++n) {   // column tile n / Kd, k-range n mod Kd
      int32_t lo, hi, klo, khi;
      tile_range(H, p.q, p.T_down / Kd, n / Kd, &lo, &hi);
      tile_range(F, 32, Kd, n % Kd, &klo, &khi);
      add(MPK_TASK_DOWN, l, n, 0, 0, {p.coarse ? full(t(L_A), F) : box(t(L_A), {0, klo}, {B, khi})},
          {box(t(L_D), {n % Kd, 0, lo}, {n % Kd + 1, B, hi})});
    }
  }
  const std::vector<Box> last = {full(layer_tensor(L - 1, L_S), H), planes(layer_tensor(L - 1, L_D), Kd, H)};
  if (!fused)
    for (int32_t b = 0; b < B; ++b) add(MPK_TASK_FINAL_NORM, -1, b, 0, 0, last, {row(T_HF, b, H)});
  for (int32_t n = 0; n < p.T_lm; ++n) {
    int32_t lo, hi;
    tile_range(V, p.q, p.T_lm, n, &lo, &hi);
    add(MPK_TASK_LMHEAD, -1, n, 0, 0, fused ? last : std::vector<Box>{full(T_HF, H)},
        {box(T_LOGITS, {0, lo}, {B, hi}), box(T_PMAX, {0, n, 0}, {B, n + 1, 2})});
  }
  add(MPK_TASK_ARGMAX, -1, 0, 0, 0, {box(T_PMAX, {0, 0, 0}, {B, p.T_lm, 2})}, {box(T_NEXT, {0}, {B})});
}

int canonicalize(const std::vector<TaskDef>& tasks, int32_t W, int jit, int fusion, Graph* out, std::string* err) {
  const int32_t N = (int32_t)tasks.size();
  if (W < 1) { *err = "n_workers must be positive"; return MPK_ERR_INVALID_ARG; }
  if (fusion != 0 && fusion != 1) { *err = "fusion order must be 0 or 1"; return MPK_ERR_UNSUPPORTED; }

  // ---- overlap dependencies: per tensor, every (out box, in box) pair with producer < consumer
  struct Ref { int32_t task; const Box* b; };
  std::map<int32_t, std::vector<Ref>> outs, ins;
  for (int32_t i = 0; i < N; ++i) {
    for (const Box& b : tasks[i].outs) outs[b.tensor].push_back({i, &b});
    for (const Box& b : tasks[i].ins) ins[b.tensor].push_back({i, &b});
  }
  std::vector<std::vector<int32_t>> P(N);
  for (auto& kv : ins) {
    auto it = outs.find(kv.first);
    if (it == outs.end()) continue;
    for (const Ref& c : kv.second)
      for (const Ref& p : it->second)
        if (p.task < c.task && overlaps(*p.b, *c.b)) P[c.task].push_back(p.task);
  }
  for (auto& v : P) {
    std::sort(v.begin(), v.end());
    v.erase(std::unique(v.begin(), v.end()), v.end());
  }

  // ---- events.  Fusion A: Def 4.1 (one event per consumer carrying all of
  //      its producers), then Def 4.2 (events with the same producer set
  //      merge, consumers unite); pre-ordered by their smallest consumer.
  //      Fusion off: one event per overlap edge (p, c), pre-ordered by (c, p).
  std::vector<std::vector<int32_t>> ev_in, ev_out;
  if (fusion == 0) {
    std::map<std::vector<int32_t>, std::vector<int32_t>> groups;
    for (int32_t c = 0; c < N; ++c)
      if (!P[c].empty()) groups[P[c]].push_back(c);
    std::vector<std::pair<std::vector<int32_t>, std::vector<int32_t>>> fused(groups.begin(), groups.end());
    std::sort(fused.begin(), fused.end(), [](const auto& a, const auto& b) { return a.second[0] < b.second[0]; });
    for (auto& f : fused) { ev_in.push_back(f.first); ev_out.push_back(f.second); }
  } else {
    for (int32_t c = 0; c < N; ++c)
      for (int32_t p : P[c]) { ev_in.push_back({p}); ev_out.push_back({c}); }
  }
  const int32_t n_fused = (int32_t)ev_in.size();
  std::vector<std::vector<int32_t>> deps_of(N), trigs_of(N);
  for (int32_t e = 0; e < n_fused; ++e) {
    for (int32_t c : ev_out[e]) deps_of[c].push_back(e);
    for (int32_t p : ev_in[e]) trigs_of[p].push_back(e);
  }

  // ---- normalisation, task by task in program order: k >= 2 dependent
  //      events (fan-in, only without fusion) -> a new event e' triggered by
  //      k empty tasks, empty i waiting on the i-th event; k >= 2 triggering
  //      events (fan-out) -> a new event e' that k empty tasks wait on, empty
  //      i triggering the i-th event.  Empties are numbered after the
  //      originals in the order they are made, coords (i, 0) for fan-out and
  //      (i, 1) for fan-in.
  std::vector<int32_t> ttype(N), tlayer(N), torig(N), dep(N, -1), trig(N, -1);
  std::vector<std::array<int32_t, 3>> tcoords(N);
  for (int32_t i = 0; i < N; ++i) {
    ttype[i] = tasks[i].type; tlayer[i] = tasks[i].layer; torig[i] = i;
    tcoords[i] = {tasks[i].c[0], tasks[i].c[1], tasks[i].c[2]};
  }
  int32_t n_empty = 0;
  auto new_empty = [&](int32_t t, int32_t i, int32_t kind) {
    const int32_t T = (int32_t)ttype.size();
    ttype.push_back(MPK_TASK_EMPTY); tlayer.push_back(tlayer[t]);
    tcoords.push_back({i, kind, 0}); torig.push_back(-1 - n_empty);
    dep.push_back(-1); trig.push_back(-1);
    ++n_empty;
    return T;
  };
  for (int32_t t = 0; t < N; ++t) {
    const std::vector<int32_t> dl = deps_of[t];
    if (dl.size() >= 2) {
      const int32_t ep = (int32_t)ev_in.size();
      ev_in.push_back({}); ev_out.push_back({t});
      for (size_t i = 0; i < dl.size(); ++i) {
        const int32_t T = new_empty(t, (int32_t)i, 1);
        dep[T] = dl[i]; trig[T] = ep;
        ev_in[ep].push_back(T);
        for (int32_t& x : ev_out[dl[i]]) if (x == t) x = T;
      }
      dep[t] = ep;
    } else if (dl.size() == 1) {
      dep[t] = dl[0];
    }
    const std::vector<int32_t> tr = trigs_of[t];
    if (tr.size() >= 2) {
      const int32_t ep = (int32_t)ev_in.size();
      ev_in.push_back({t}); ev_out.push_back({});
      for (size_t i = 0; i < tr.size(); ++i) {
        const int32_t T = new_empty(t, (int32_t)i, 0);
        dep[T] = ep; trig[T] = tr[i];
        ev_out[ep].push_back(T);
        for (int32_t& x : ev_in[tr[i]]) if (x == t) x = T;
      }
      trig[t] = ep;
    } else if (tr.size() == 1) {
      trig[t] = tr[0];
    }
  }
  const int32_t NT = (int32_t)ttype.size();
  const int32_t root = (int32_t)ev_in.size();
  ev_in.push_back({}); ev_out.push_back({});
  const int32_t end = (int32_t)ev_in.size();
  ev_in.push_back({}); ev_out.push_back({});
  for (int32_t t = 0; t < NT; ++t) {
    if (dep[t] < 0) { dep[t] = root; ev_out[root].push_back(t); }
    if (trig[t] < 0) { trig[t] = end; ev_in[end].push_back(t); }
  }
  const int32_t NE = (int32_t)ev_in.size();

  // ---- Kahn-BFS linearisation: an event is enqueued when its last producer
  //      is placed; a dequeued event places its consumers consecutively.
  std::vector<int32_t> indeg(NE), new_ev(NE, -1), new_task(NT, -1), first(NE, 0), last(NE, 0);
  for (int32_t e = 0; e < NE; ++e) indeg[e] = (int32_t)ev_in[e].size();
  std::deque<int32_t> q{root};
  int32_t ne = 0, nt = 0;
  while (!q.empty()) {
    int32_t e = q.front();
    q.pop_front();
    new_ev[e] = ne++;
    first[e] = nt;
    std::vector<int32_t> o = ev_out[e];
    std::sort(o.begin(), o.end());
    for (int32_t t : o) {
      new_task[t] = nt++;
      int32_t f = trig[t];
      if (--indeg[f] == 0) q.push_back(f);
    }
    last[e] = nt - 1;
  }
  if (nt != NT || ne != NE) { *err = "tGraph has a cycle"; return MPK_ERR_GRAPH; }

  Graph& g = *out;
  g = Graph();
  g.NT = NT; g.NE = NE; g.root = new_ev[root]; g.end = new_ev[end];
  g.n_fused = n_fused; g.n_empty = n_empty; g.n_rewrites = NE - 2 - n_fused;
  std::vector<int32_t> order(NT), eorder(NE);
  for (int32_t t = 0; t < NT; ++t) order[new_task[t]] = t;
  for (int32_t e = 0; e < NE; ++e) eorder[new_ev[e]] = e;
  // (JIT tasks are handed over when their event fires; the root event is
  // never triggered, so its consumers stay AOT under every policy)
  // (attention splits and expert tiles are the tasks whose work is decided by
  // data when the step runs: JIT under the hybrid policy)
  auto mode_of = [jit, root](int32_t type, int32_t dep_ev) {
    const bool dd = type == MPK_TASK_ATTN || type == MPK_TASK_EXPERT_GU || type == MPK_TASK_EXPERT_DOWN;
    return type == MPK_TASK_EMPTY                                   ? MPK_MODE_EMPTY
           : dep_ev != root && (jit == 2 || (dd && jit == 1)) ? MPK_MODE_JIT
                                                                    : MPK_MODE_AOT;
  };
  g.task_type.resize(NT); g.task_mode.resize(NT); g.task_layer.resize(NT); g.task_coords.resize(3 * (size_t)NT);
  g.task_orig.resize(NT); g.task_dep.resize(NT); g.task_trig.resize(NT); g.task_worker.assign(NT, -1);
  for (int32_t i = 0; i < NT; ++i) {
    int32_t t = order[i];
    g.task_type[i] = (uint8_t)ttype[t];
    g.task_mode[i] = (uint8_t)mode_of(ttype[t], dep[t]);
    g.task_layer[i] = (int16_t)tlayer[t];
    for (int k = 0; k < 3; ++k) g.task_coords[3 * (size_t)i + k] = (uint16_t)tcoords[t][k];
    g.task_orig[i] = torig[t];
    g.task_dep[i] = new_ev[dep[t]];
    g.task_trig[i] = new_ev[trig[t]];
  }
  g.event_counts.resize(NE); g.event_first.resize(NE); g.event_last.resize(NE); g.event_flags.assign(NE, 0);
  for (int32_t i = 0; i < NE; ++i) {
    int32_t e = eorder[i];
    g.event_counts[i] = (uint32_t)ev_in[e].size();
    g.event_first[i] = first[e];
    g.event_last[i] = last[e];
    for (int32_t t : ev_out[e]) {
      int m = mode_of(ttype[t], e);
      if (m == MPK_MODE_JIT) g.event_flags[i] |= MPK_EVENT_HAS_JIT;
      if (m == MPK_MODE_EMPTY) g.event_flags[i] |= MPK_EVENT_HAS_EMPTY;
    }
  }
  // ---- AOT placement: round-robin over workers in linear order
  std::vector<std::vector<uint32_t>> lists(W);
  int64_t k = 0;
  for (int32_t i = 0; i < NT; ++i) {
    if (g.task_mode[i] != MPK_MODE_AOT) continue;
    int32_t w = (int32_t)(k % W);
    g.task_worker[i] = (int16_t)w;
    lists[w].push_back((uint32_t)i);
    ++k;
  }
  g.aot_offsets.assign(W + 1, 0);
  for (int32_t w = 0; w < W; ++w) {
    g.aot_offsets[w + 1] = g.aot_offsets[w] + (uint32_t)lists[w].size();
    g.aot_tasks.insert(g.aot_tasks.end(), lists[w].begin(), lists[w].end());
  }
  return MPK_OK;
}

}  // namespace mpk
